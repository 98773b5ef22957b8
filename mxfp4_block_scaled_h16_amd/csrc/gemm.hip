// Block-scaled MXFP4 GEMM on gfx950's scaled FP4 matrix cores, FP32 accumulate and output.
//
// The MXFP4 GEMMs of the gist.science summary of "MXFP4 LLM pretraining", section 방법론
// (Methodology), run natively on the FP4 matrix cores: c[m][n] = alpha * sum_k deq(A)[m][k] *
// deq(B)[n][k] with both operands quantized along K (32-element blocks, one E8M0 byte each).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both formats E2M1: each lane supplies 32 K-consecutive
// codes (16 bytes) of one row of A and of one row of B -- exactly one MX block -- plus that
// block's scale byte; lane l holds row (l % 32) and K-half (l / 32) of the 32 x 64 step. The
// 32 x 32 FP32 result sits in 16 registers per lane: register i of lane l is row
// 8 (i / 4) + 4 (l / 32) + (i % 4), column l % 32.
#include <climits>

#include "internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kFmtFp4 = 4;  // format selector of the f8f6f4 MFMA family for E2M1

// Workgroup tile 128 x 128, four wavefronts in a 2 x 2 arrangement, each 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32); one K step = 64 (two MX blocks per row).
constexpr int kTileM = 128, kTileN = 128, kWaveM = 64, kWaveN = 64;

__global__ __launch_bounds__(256) void gemm_mxfp4_simple(
    const uint8_t *__restrict__ aq, int64_t lda, const uint8_t *__restrict__ as, int64_t ldas,
    const uint8_t *__restrict__ bq, int64_t ldb, const uint8_t *__restrict__ bs, int64_t ldbs,
    int M, int N, int K, float alpha, float *__restrict__ c, int64_t ldc)
{
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m_base = blockIdx.y * kTileM + (wave >> 1) * kWaveM;
    const int n_base = blockIdx.x * kTileN + (wave & 1) * kWaveN;
    const int r = lane & 31;
    const int half = lane >> 5;

    const uint8_t *pa[2], *psa[2], *pb[2], *psb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int row_a = min(m_base + 32 * i + r, M - 1);
        const int row_b = min(n_base + 32 * i + r, N - 1);
        pa[i] = aq + (int64_t)row_a * lda + 16 * half;
        psa[i] = as + (int64_t)row_a * ldas + half;
        pb[i] = bq + (int64_t)row_b * ldb + 16 * half;
        psb[i] = bs + (int64_t)row_b * ldbs + half;
    }

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += 64) {
        // the second half of the last step is past K when K is an odd multiple of 32
        const bool live = k0 + 32 * half < K;
        v8i fa[2], fb[2];
        int sa[2], sb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            uint4 ta = make_uint4(0, 0, 0, 0), tb = make_uint4(0, 0, 0, 0);
            int xa = 127, xb = 127;
            if (live) {
                ta = *reinterpret_cast<const uint4 *>(pa[i] + k0 / 2);
                tb = *reinterpret_cast<const uint4 *>(pb[i] + k0 / 2);
                xa = psa[i][k0 / 32];
                xb = psb[i][k0 / 32];
            }
            fa[i] = v8i{(int)ta.x, (int)ta.y, (int)ta.z, (int)ta.w, 0, 0, 0, 0};
            fb[i] = v8i{(int)tb.x, (int)tb.y, (int)tb.z, (int)tb.w, 0, 0, 0, 0};
            sa[i] = xa;
            sb[i] = xb;
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    fa[i], fb[j], acc[i][j], kFmtFp4, kFmtFp4, 0, sa[i], 0, sb[j]);
    }

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n_base + 32 * j + r;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m_base + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
                if (m < M) c[(int64_t)m * ldc + n] = alpha * acc[i][j][e];
            }
        }
}

// ------------------------------------------------------------------------------------------
// Tiled kernel: 256 x 256 workgroup tile, four wavefronts of 128 x 128 (4 x 4 MFMA tiles, 256
// accumulator registers each, one wavefront per SIMD). Operand codes move HBM -> LDS by direct
// 16-byte-per-lane DMA (global_load_lds_dwordx4), double-buffered over K stages of 256 values
// (128 bytes per row). Rows are stored with their 16-byte chunks XOR-swizzled so that the
// fragment reads (ds_read_b128, one MX block per lane) hit distinct banks. Scale bytes go straight
// from memory into registers (8 per row and stage), shifted per lane so the MFMA's byte selector
// is the same for the whole wavefront.
// Requirements (checked by the dispatcher): K % 256 == 0, scales rows 8-byte aligned.

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

constexpr int kBM = 256, kBN = 256;
constexpr int kRowBytes = 128;                  // codes per row per stage (256 E2M1 values)
constexpr int kStageK = 2 * kRowBytes;          // K values per stage
constexpr int kABytes = kBM * kRowBytes;        // 32 KB
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;  // 64 KB
constexpr int kRowsPerDma = 1024 / kRowBytes;   // one wave-wide 16 B/lane DMA covers 8 rows
constexpr int kDmaPerWave = kBM / kRowsPerDma / 4;  // 8 per operand per wavefront

// chunk permutation of a row: rows r..r+7 and every other row of r..r+15 all land in distinct
// 16-byte bank groups when the same logical chunk is read
__device__ __forceinline__ int chunk_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

__device__ __forceinline__ void mfma_tile(v16f &acc, const u32x4 &a, const u32x4 &b, int sa, int sb,
                                          int opsel_hi)
{
    const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    if (opsel_hi)
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, kFmtFp4, kFmtFp4, 2, sa, 2, sb);
    else
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, vb, acc, kFmtFp4, kFmtFp4, 0, sa, 0, sb);
}

__global__ __launch_bounds__(256, 1) void gemm_mxfp4_tiled(
    const uint8_t *__restrict__ aq, int64_t lda, const uint8_t *__restrict__ as, int64_t ldas,
    const uint8_t *__restrict__ bq, int64_t ldb, const uint8_t *__restrict__ bs, int64_t ldbs,
    int M, int N, int K, float alpha, float *__restrict__ c, int64_t ldc, int tiles_m, int tiles_n)
{
    __shared__ __attribute__((aligned(1024))) uint8_t lds[2 * kStageBytes];

    // tile order: consecutive workgroups are spread over the 8 XCDs; give each XCD a contiguous
    // range of tiles, walked column-panel by column-panel in groups of 8 row panels
    const int total = tiles_m * tiles_n;
    int t = blockIdx.x;
    if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
    const int group = 8 * tiles_n;
    const int g0 = (t / group) * 8;
    const int gm = min(8, tiles_m - g0);
    const int tm = g0 + (t % group) % gm;
    const int tn = (t % group) / gm;
    const int m0 = tm * kBM, n0 = tn * kBN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 31, half = lane >> 5;
    const int swz = chunk_swizzle(r);

    // DMA sources: instruction (wave, t) fills LDS rows [8 (8 wave + t), + 8); lane L writes the
    // 16 bytes at row 8 (8 wave + t) + L / 8, physical chunk L % 8 = logical chunk ^ swizzle
    uint32_t a_off[kDmaPerWave], b_off[kDmaPerWave];
#pragma unroll
    for (int u = 0; u < kDmaPerWave; ++u) {
        const int row = kRowsPerDma * (kDmaPerWave * wave + u) + lane / 8;
        const int chunk = (lane % 8) ^ chunk_swizzle(row);
        a_off[u] = (uint32_t)(min(m0 + row, M - 1) * lda + 16 * chunk);
        b_off[u] = (uint32_t)(min(n0 + row, N - 1) * ldb + 16 * chunk);
    }
    // scale sources of this lane's fragment rows
    const uint8_t *sa_ptr[4], *sb_ptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sa_ptr[i] = as + (int64_t)min(m0 + wm * 128 + 32 * i + r, M - 1) * ldas;
        sb_ptr[i] = bs + (int64_t)min(n0 + wn * 128 + 32 * i + r, N - 1) * ldbs;
    }

    auto dma_stage = [&](int buf, int kstage) {
        uint8_t *dst = lds + buf * kStageBytes;
        const int kb = kstage * kRowBytes;
#pragma unroll
        for (int u = 0; u < kDmaPerWave; ++u) {
            const int row0 = kRowsPerDma * (kDmaPerWave * wave + u);
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(aq + a_off[u] + kb),
                                             (lds_void_t *)(dst + row0 * kRowBytes), 16, 0, 0);
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(bq + b_off[u] + kb),
                                             (lds_void_t *)(dst + kABytes + row0 * kRowBytes), 16, 0, 0);
        }
    };
    // 8 scale bytes per fragment row and stage, kept raw until the stage is computed (shifting
    // them at load time would make the wavefront wait for the loads just issued)
    auto load_scales = [&](int kstage, uint64_t (&sa)[4], uint64_t (&sb)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = *reinterpret_cast<const uint64_t *>(sa_ptr[i] + 8 * kstage);
            sb[i] = *reinterpret_cast<const uint64_t *>(sb_ptr[i] + 8 * kstage);
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int nk = K / kStageK;
    uint64_t sa_raw[4], sb_raw[4], sa_nxt[4], sb_nxt[4];
    dma_stage(0, 0);
    load_scales(0, sa_raw, sb_raw);

    const int a_row0 = wm * 128 + r;
    const int b_row0 = wn * 128 + r;
    for (int ks = 0; ks < nk; ++ks) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this stage's DMA and scales landed
        __syncthreads();                      // ... for every wavefront; the other buffer is free
        // byte 0 / byte 2 of each word = this lane's block for even / odd K64 sub-steps
        uint32_t sa[4][2], sb[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i][0] = (uint32_t)sa_raw[i] >> (8 * half);
            sa[i][1] = (uint32_t)(sa_raw[i] >> 32) >> (8 * half);
            sb[i][0] = (uint32_t)sb_raw[i] >> (8 * half);
            sb[i][1] = (uint32_t)(sb_raw[i] >> 32) >> (8 * half);
        }
        if (ks + 1 < nk) {
            dma_stage((ks + 1) & 1, ks + 1);
            load_scales(ks + 1, sa_nxt, sb_nxt);
        }
        const uint8_t *sbuf = lds + (ks & 1) * kStageBytes;
        // fragments of sub-step kk + 1 are read while the 16 MFMAs of sub-step kk run
        u32x4 fa[2][4], fb[2][4];
        auto read_frags = [&](int kk, u32x4 (&a)[4], u32x4 (&b)[4]) {
            const int chunk = (2 * kk + half) ^ swz;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = *reinterpret_cast<const u32x4 *>(sbuf + (a_row0 + 32 * i) * kRowBytes + 16 * chunk);
                b[i] = *reinterpret_cast<const u32x4 *>(sbuf + kABytes + (b_row0 + 32 * i) * kRowBytes + 16 * chunk);
            }
        };
        read_frags(0, fa[0], fb[0]);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int cur = kk & 1;
            if (kk < 3) read_frags(kk + 1, fa[cur ^ 1], fb[cur ^ 1]);
            __builtin_amdgcn_sched_barrier(0);  // the reads above are issued before these MFMAs
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    mfma_tile(acc[i][j], fa[cur][i], fb[cur][j], (int)sa[i][kk >> 1], (int)sb[j][kk >> 1],
                              kk & 1);
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa_raw[i] = sa_nxt[i];
            sb_raw[i] = sb_nxt[i];
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 128 + 32 * j + r;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (e / 4) + 4 * half + (e % 4);
                if (m < M) c[(int64_t)m * ldc + n] = alpha * acc[i][j][e];
            }
        }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float *__restrict__ c, int64_t M, int64_t N,
                                                       int64_t ldc)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < M * N) c[(i / N) * ldc + (i % N)] = 0.0f;
}

}  // namespace

hipError_t launch_fill_zero(float *c, int64_t M, int64_t N, int64_t ldc, hipStream_t stream)
{
    const int64_t total = M * N;
    if (total == 0) return hipSuccess;
    return launch(fill_zero_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream, c, M,
                  N, ldc);
}

hipError_t launch_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                       const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs, int64_t M,
                       int64_t N, int64_t K, float alpha, float *c, int64_t ldc, hipStream_t stream)
{
    const bool scales_aligned = ((uintptr_t)as % 8 == 0) && ((uintptr_t)bs % 8 == 0) && ldas % 8 == 0 &&
                                ldbs % 8 == 0;
    const bool offsets_fit = (int64_t)(M - 1) * lda + lda <= INT32_MAX && (int64_t)(N - 1) * ldb + ldb <= INT32_MAX;
    if (K % kStageK == 0 && K > 0 && scales_aligned && offsets_fit) {
        const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
        return launch(gemm_mxfp4_tiled, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0, stream, aq,
                      lda, as, ldas, bq, ldb, bs, ldbs, (int)M, (int)N, (int)K, alpha, c, ldc, tiles_m,
                      tiles_n);
    }
    const dim3 grid((unsigned)((N + kTileN - 1) / kTileN), (unsigned)((M + kTileM - 1) / kTileM));
    return launch(gemm_mxfp4_simple, grid, dim3(256), 0, stream, aq, lda, as, ldas, bq, ldb, bs, ldbs,
                  (int)M, (int)N, (int)K, alpha, c, ldc);
}

}  // namespace mx

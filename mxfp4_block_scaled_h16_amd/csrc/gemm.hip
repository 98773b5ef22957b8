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
    const dim3 grid((unsigned)((N + kTileN - 1) / kTileN), (unsigned)((M + kTileM - 1) / kTileM));
    return launch(gemm_mxfp4_simple, grid, dim3(256), 0, stream, aq, lda, as, ldas, bq, ldb, bs, ldbs,
                  (int)M, (int)N, (int)K, alpha, c, ldc);
}

}  // namespace mx

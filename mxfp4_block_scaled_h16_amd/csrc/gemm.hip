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
#include <type_traits>

#include "internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kFmtFp4 = 4;  // format selector of the f8f6f4 MFMA family for E2M1

// ------------------------------------------------------------------ accumulation chains -----
// A scaled FP4 MFMA adds its block products (one per 32 K values: an exact integer times a power
// of two) to the FP32 accumulator one at a time, in K order, rounding to nearest even after each
// (GPU tests pin this: 1 followed by two blocks of 0.375 units in the last place stays 1, while
// the same blocks before the 1 round it up). So an output accumulated in a single chain over K
// values has gone through up to K / 32 roundings, and a term that passes through D roundings
// carries a relative error of at most D u / (1 - D u), u = 2^-24. Every output meets
// |c - c_exact| <= 1e-5 * sum_k |a_k b_k| as long as no term goes through more than
// kMaxDepth = 167 roundings, i.e. K <= 5344 in one chain; a worst case reaches the bound (a
// chain stuck at 1 while every later block adds just under half a unit in the last place).
// Longer contractions are cut into segments: each segment accumulates from zero, and the
// segments are added in their K order, which puts a term through at most (segment blocks) +
// (number of segments) roundings. Split-K partials obey the same count.
constexpr int kMaxDepth = 167;

// Length, in units of `per_unit` blocks, of the segments that a chain of `units` units is cut
// into; 0 when the whole chain is within the bound. Segments are as long as the bound allows for
// the fewest of them; past about 7000 blocks (K of about 220 thousand) no two-level split meets
// it, and the shortest segments are returned.
int chain_segment(int64_t units, int per_unit)
{
    if (units * per_unit + 1 <= kMaxDepth) return 0;
    for (int64_t c = 2; c <= units; ++c) {
        const int64_t per = (units + c - 1) / c;
        const int64_t segs = (units + per - 1) / per;
        if (per * per_unit + segs <= kMaxDepth) return (int)per;
    }
    return 1;
}

// ---------------------------------------------------------------------------- output ---------
// The general epilogue: c = alpha * (A B^T) + beta * c, stored as FP32 or bf16 (the FP32 value
// rounded to nearest even by the hardware conversion). c is read only when beta != 0 (it may be
// uninitialised otherwise).
struct OutSpec {
    void *c;
    int64_t ldc;
    float alpha, beta;
    int bf16;
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b)
{
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// one output element (v = alpha * acc already)
template <bool BF16>
__device__ __forceinline__ void store1(const OutSpec &o, int64_t m, int64_t n, float v)
{
    if constexpr (BF16) {
        uint16_t *p = static_cast<uint16_t *>(o.c) + m * o.ldc + n;
        if (o.beta != 0.0f) v = v + o.beta * bf16_bits_to_float(*p);
        *p = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
    } else {
        float *p = static_cast<float *>(o.c) + m * o.ldc + n;
        if (o.beta != 0.0f) v = v + o.beta * *p;
        *p = v;
    }
}

__device__ __forceinline__ void store1_any(const OutSpec &o, int64_t m, int64_t n, float v)
{
    if (o.bf16)
        store1<true>(o, m, n, v);
    else
        store1<false>(o, m, n, v);
}

// four consecutive outputs (v = alpha * acc already); vec: the row segment is aligned for one
// 16-byte (FP32) or 8-byte (bf16) access and lies inside [0, N)
template <bool BF16>
__device__ __forceinline__ void store4(const OutSpec &o, int64_t m, int64_t n, int64_t N, f32x4v v, bool vec)
{
    if (!vec) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (n + e < N) store1<BF16>(o, m, n + e, v[e]);
        return;
    }
    if constexpr (BF16) {
        uint2 *p = reinterpret_cast<uint2 *>(static_cast<uint16_t *>(o.c) + m * o.ldc + n);
        if (o.beta != 0.0f) {
            const uint2 old = *p;
            v[0] = v[0] + o.beta * bf16_bits_to_float(old.x & 0xFFFFu);
            v[1] = v[1] + o.beta * bf16_bits_to_float(old.x >> 16);
            v[2] = v[2] + o.beta * bf16_bits_to_float(old.y & 0xFFFFu);
            v[3] = v[3] + o.beta * bf16_bits_to_float(old.y >> 16);
        }
        *p = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
    } else {
        f32x4v *p = reinterpret_cast<f32x4v *>(static_cast<float *>(o.c) + m * o.ldc + n);
        if (o.beta != 0.0f) v = v + o.beta * *p;
        *p = v;
    }
}

// the row segments of c starting at column n (a multiple of 4) allow vector accesses
template <bool BF16>
__device__ __forceinline__ bool out_vector_ok(const OutSpec &o)
{
    return (o.ldc % 4) == 0 && ((uintptr_t)o.c % (BF16 ? 8 : 16)) == 0;
}

// epilogue variants of the pipelined kernel
constexpr int kEpiF32 = 0;      // c = alpha * A B^T, FP32 (nothing else compiled in)
constexpr int kEpiF32Beta = 1;  // FP32 with beta
constexpr int kEpiBF16 = 2;     // bf16 with beta

// Workgroup tile 128 x 128, four wavefronts in a 2 x 2 arrangement, each 64 x 64 (2 x 2 MFMA
// tiles of 32 x 32); one K step = 64 (two MX blocks per row).
constexpr int kTileM = 128, kTileN = 128, kWaveM = 64, kWaveN = 64;
constexpr int kGroupMax = 8;                          // products of one grouped launch

// The products of a grouped launch: same shapes, strides and layout, operands and outputs of
// their own.
struct GroupItem {
    const uint8_t *aq, *as, *bq, *bs;
    float *c;
};
struct GroupArgs {
    GroupItem item[kGroupMax];
    int count;
};

// FOLD: the accumulation chain restarts from zero every fold_steps MFMA steps, the finished
// segments summed in K order in a second set of registers (contractions longer than one chain
// may be). A grouped launch (grp.count > 0) runs product blockIdx.z of grp.
template <bool FOLD>
__global__ __launch_bounds__(256) void gemm_mxfp4_simple(
    const uint8_t *__restrict__ aq, int64_t lda, const uint8_t *__restrict__ as, int64_t ldas,
    const uint8_t *__restrict__ bq, int64_t ldb, const uint8_t *__restrict__ bs, int64_t ldbs,
    int M, int N, int K, OutSpec out, int fold_steps, GroupArgs grp)
{
    if (grp.count > 0) {
        const GroupItem &it = grp.item[blockIdx.z];
        aq = it.aq;
        as = it.as;
        bq = it.bq;
        bs = it.bs;
        out.c = it.c;
    }
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

    v16f acc[2][2], seg_sum[FOLD ? 2 : 1][FOLD ? 2 : 1];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    if constexpr (FOLD) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) seg_sum[i][j] = v16f{};
    }

    for (int k0 = 0, step = 1; k0 < K; k0 += 64, ++step) {
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
        if constexpr (FOLD) {
            // end of a segment of the accumulation chain (not after the last step)
            if (step % fold_steps == 0 && k0 + 64 < K) {
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        seg_sum[i][j] = seg_sum[i][j] + acc[i][j];
                        acc[i][j] = v16f{};
                    }
            }
        }
    }
    if constexpr (FOLD) {
        // the last segment joins the earlier ones
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) acc[i][j] = seg_sum[i][j] + acc[i][j];
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
                if (m < M) store1_any(out, m, n, out.alpha * acc[i][j][e]);
            }
        }
}

// ------------------------------------------------------------------------------------------
// Pipelined kernel: 256 x 256 workgroup tile, eight wavefronts of 128 x 64 (4 x 2 MFMA tiles,
// 128 accumulator registers each, two wavefronts per SIMD: while one waits for its operands the
// other issues MFMAs). The four-wavefront form (128 x 128 each, one per SIMD) is the other
// instantiation; eight measured 2-3% faster per step once the output went through LDS.
//
// The MFMA pipe of a SIMD only stays busy if its wavefronts keep issuing, so the K loop is
// software-pipelined around them:
//  * operand codes move HBM -> LDS by direct 16-byte-per-lane DMA into a ring of four stage
//    buffers of 128 K values (64 bytes per row), issued three stages ahead; each wait is for the
//    oldest stage only (vmcnt with the exact number of younger loads);
//  * scale bytes move the same way, 16 per row (four stages) at a time, into two LDS slots;
//  * LDS fragment and scale reads for the next 64-wide sub-step are issued between the MFMAs of
//    the current one, and so are the DMA instructions;
//  * the product is formed transposed (B as the MFMA's first operand), so each lane ends with
//    four consecutive output columns per register quad;
//  * the epilogue stages each wavefront's result through LDS in 32-row slices, so that every
//    store instruction writes whole row segments (whole 128-byte lines) instead of 32-byte
//    pieces of 32 rows: the FP32 output is the largest HBM stream of the kernel and its writes
//    all come at once, when every CU finishes its tile;
//  * with more tiles than CUs, one workgroup per CU walks them (the PERSIST form below): the
//    next tile's first two stages and scales are loaded during the current tile's last stages,
//    so a CU's later tiles start without a prologue and its stores drain during the next
//    tile's first stage.
// Rows of a stage buffer hold their four 16-byte chunks XOR-permuted by bits 2-3 of the row: the
// LDS serves a 16-byte-per-lane read 16 lanes (256 bytes, 64 banks) at a time, and the 16 rows
// those lanes read then land in 16 distinct bank groups.
// Requirements (checked by the dispatcher): K % 512 == 0; scale rows 16-byte aligned; row byte
// offsets fit in 32 bits.

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef const __attribute__((address_space(1))) void gbl_void_t;

constexpr int kBM = 256, kBN = 256;                  // the main workgroup tile
constexpr int kStageK = 128;                          // K values per stage
constexpr int kRowBytes = kStageK / 2;                // 64 bytes of codes per row per stage
constexpr int kNumBuf = 4;                            // stage ring; a group = 4 stages
constexpr int kRowsPerDma = 1024 / kRowBytes;         // one wave-wide 16 B/lane DMA covers 16 rows
constexpr int kGemmWaves = 8;                         // wavefronts per workgroup (4 or 8)
// the tile of products whose contraction needs a segmented accumulation chain: 256 x 128, eight
// wavefronts of 64 x 64 (a 128 x 64 wave tile has no registers left for the second accumulator
// set). Measured against four wavefronts of 128 x 64 (one per SIMD, 455 registers): the same
// (gate Dgrad 8192 x 4096 x 14336: 271.7 vs 276.8 us); 128 x 128 tiles: 285 us.
constexpr int kFoldWaves = 8, kFoldTM = 256, kFoldTN = 128;
constexpr int kComputeUnits = 256;                    // MI355X

__device__ __forceinline__ int chunk_perm(int row) { return (row >> 2) & 3; }

template <int OPSEL>
__device__ __forceinline__ void mfma_t(v16f &acc, const u32x4 &b, const u32x4 &a, uint32_t sb, uint32_t sa)
{
    const v8i vb = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const v8i va = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vb, va, acc, kFmtFp4, kFmtFp4, OPSEL, (int)sb,
                                                          OPSEL, (int)sa);
}

// s_waitcnt vmcnt(N) with N < 64 (gfx9 encoding: low 4 bits in [3:0], high 2 bits in [15:14];
// expcnt and lgkmcnt fields left at their "no wait" maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Geometry of the pipelined kernel: NW wavefronts, a TM x TN workgroup tile (TM rows of A, TN
// rows of B), the wavefronts arranged WM x (NW / WM) with wave tiles of TM / WM rows (FI 32-row
// MFMA tiles of A) by TN WM / NW columns (FJ 32-column tiles of B). Instantiated as:
//  * 256 x 256, eight wavefronts of 128 x 64: the main tile (one workgroup per CU);
//  * 128 x 128, four wavefronts of 64 x 64: products with fewer 256 x 256 tiles than half the
//    CUs (half the LDS, two workgroups per CU);
//  * 256 x 128, eight wavefronts of 64 x 64: contractions that need a segmented accumulation
//    chain, whose second set of accumulators does not fit the main tile's wavefronts.
template <int NW, int TM, int TN, int WM>
struct Geo {
    static_assert(TM % 64 == 0 && TN % 64 == 0 && NW % WM == 0, "pipelined geometries");
    static constexpr int kTileM = TM, kTileN = TN;
    static constexpr int kABytes = TM * kRowBytes;                // 16 KB for TM = 256
    static constexpr int kStageBytes = (TM + TN) * kRowBytes;     // 32 KB for 256 x 256
    static constexpr int kScaleSlot = (TM + TN) * 16;             // 16 scale bytes per row per group
    static constexpr int kScaleBase = kNumBuf * kStageBytes;      // two scale slots after the stage ring
    static constexpr int kLdsBytes = kScaleBase + 2 * kScaleSlot; // 144 KB for 256 x 256
    static constexpr int kWavesM = WM, kWavesN = NW / WM;
    static constexpr int kWaveRows = TM / kWavesM;
    static constexpr int kWaveCols = TN / kWavesN;
    static constexpr int FI = kWaveRows / 32, FJ = kWaveCols / 32;
    static constexpr int kDmaA = TM / kRowsPerDma / NW;           // per wavefront and stage
    static constexpr int kDmaB = TN / kRowsPerDma / NW;
    static_assert(kDmaA * kRowsPerDma * NW == TM && kDmaB * kRowsPerDma * NW == TN, "whole DMAs per wavefront");
    static constexpr int kDmaPerStage = kDmaA + kDmaB;
    static constexpr int kScaleChunks = (TM + TN) / 64;           // 64-row scale DMAs per group
    static constexpr int kDmaPerScales = (kScaleChunks + NW - 1) / NW;  // per wavefront and group
    static constexpr int kMinBlocks = kLdsBytes <= 80 * 1024 ? 2 : 1;   // workgroups per CU
};

// where a virtual block of the pipelined kernel works: its K-split, tile origin, operands, output
struct TileWhere {
    int split, m0, n0;
    const uint8_t *aq, *as, *bq, *bs;
    void *c;
};
// a lane's DMA source offsets for one tile: codes of A and B, scales (and their operand)
template <int DA, int DB, int DS>
struct DmaOffsets {
    uint32_t a[DA], b[DB], s[DS];
    const uint8_t *src[DS];
};

// EPI: kEpiF32 writes FP32 c = alpha * A B^T (out.c a float pointer; no other epilogue code is
// compiled in), kEpiF32Beta adds beta * c, kEpiBF16 writes bf16 (with beta * c).
// GROUP: the grid covers grp.count products (FP32 output, no split of K), one after another in
// blockIdx order before the spread over the XCDs, so their tiles fill the chip together.
// FOLD: the accumulation chain restarts from zero every fold_groups groups of four stages, the
// finished segments summed in K order in a second set of registers (contractions longer than
// one chain may be; only geometries with 64 x 64 wave tiles have the registers for it).
// PERSIST: a grid of at most one workgroup per CU walks the tiles (virtual block blockIdx.x, then
// + gridDim.x, ...), and the first two stages and scales of its next tile are loaded during the
// last stages of the current one (FP32 output, unsplit, an even number of groups).
template <int NW, bool TILED, int EPI, int TM = kBM, int TN = kBN, int WM = 2, bool FOLD = false, bool GROUP = false,
          bool PERSIST = false>
__global__ __launch_bounds__(64 * NW, (Geo<NW, TM, TN, WM>::kMinBlocks)) void gemm_mxfp4_pipelined(
    const uint8_t *__restrict__ aq, int64_t lda, const uint8_t *__restrict__ as, int64_t ldas,
    const uint8_t *__restrict__ bq, int64_t ldb, const uint8_t *__restrict__ bs, int64_t ldbs,
    int M, int N, int K, OutSpec out, int tiles_m, int tiles_n, int splits, float *__restrict__ partials,
    int fold_groups, GroupArgs grp)
{
    static_assert(!GROUP || EPI == kEpiF32, "grouped products write FP32 without beta");
    using G = Geo<NW, TM, TN, WM>;
    static_assert(!FOLD || G::FI * G::FJ <= 4, "segmented accumulation needs wave tiles of at most 64 x 64");
    static_assert(!PERSIST || EPI == kEpiF32, "the persistent walk writes FP32 without beta");
    constexpr int FI = G::FI, FJ = G::FJ;
    constexpr int kABytes = G::kABytes, kStageBytes = G::kStageBytes, kScaleSlot = G::kScaleSlot;
    // LDS: the stage ring, then the two scale slots. The walk puts the scale slots first, so that
    // ring buffers 2 and 3 and the space after them hold the epilogue's 32-row slices (unpadded,
    // one per wavefront) while the next tile's first stages land in buffers 0 and 1.
    constexpr int kRingBase = PERSIST ? 2 * kScaleSlot : 0;
    constexpr int kScaleBase = PERSIST ? 0 : G::kScaleBase;
    constexpr int kSliceOut = kRingBase + 2 * kStageBytes;
    constexpr int kWalkLds = kSliceOut + NW * 32 * G::kWaveCols * 4;
    constexpr int kLdsBytes = PERSIST && kWalkLds > G::kLdsBytes ? kWalkLds : G::kLdsBytes;
    static_assert(kLdsBytes <= 160 * 1024, "LDS of one CU");
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kLdsBytes];

    // tile order: consecutive workgroups are spread over the 8 XCDs; give each XCD a contiguous
    // range of tiles, walked column-panel by column-panel in groups of row panels covering 1024
    // rows of A, so that one round of an XCD's 32 CUs shares its operand panels through that
    // XCD's L2: 4 row panels x 8 column panels of 256 x 128 tiles (20% fewer operand bytes per
    // round than 8 x 4; 1-1.5% faster on the segmented-chain products of the decoder layer), and
    // 4 x 8 of 256 x 256 tiles too (with the tile walk, 2-5% faster than 8 x 4 on the layer's
    // 256 x 256 products in two same-session A/Bs, 16 x 2 slower)
    const int total = tiles_m * tiles_n;
    constexpr int kGroupRows = 1024 / TM;
    // virtual block v: its K-split, tile origin and (grouped) the product's operands and output
    auto locate = [&](int v) {
        TileWhere w;
        int t;
        if constexpr (GROUP) {
            // the products' tiles as one range spread over the XCDs, product by product
            const int all = total * grp.count;
            int u = v;
            if (all % 8 == 0) u = (u % 8) * (all / 8) + u / 8;
            const int gi = u / total;
            t = u % total;
            w.split = 0;
            w.aq = grp.item[gi].aq;
            w.as = grp.item[gi].as;
            w.bq = grp.item[gi].bq;
            w.bs = grp.item[gi].bs;
            w.c = grp.item[gi].c;
        } else {
            // split-K: block v covers K-split v / total of tile v % total (the walk never splits)
            w.split = PERSIST ? 0 : v / total;
            t = PERSIST ? v : v % total;
            if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;
            w.aq = aq;
            w.as = as;
            w.bq = bq;
            w.bs = bs;
            w.c = out.c;
        }
        const int group = kGroupRows * tiles_n;
        const int g0 = (t / group) * kGroupRows;
        const int gm = min(kGroupRows, tiles_m - g0);
        w.m0 = (g0 + (t % group) % gm) * TM;
        w.n0 = ((t % group) / gm) * TN;
        return w;
    };
    int vblock = blockIdx.x;
    TileWhere cur = locate(vblock);
    int split = cur.split, m0 = cur.m0, n0 = cur.n0;
    aq = cur.aq;
    bq = cur.bq;
    out.c = cur.c;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % G::kWavesM, wn = wave / G::kWavesM;
    const int r = lane & 31, half = lane >> 5;

    // code DMA: instruction u of this wavefront fills stage rows [16 (kDmaA wave + u), + 16) of A
    // (and likewise with kDmaB of B); lane L writes the 16 bytes at row + L / 4, physical chunk
    // L % 4. Row-major operands: lane L reads its row's logical chunk (L % 4) ^ perm(row). Tiled
    // operands already hold each 16-row x 128-K block as those 1024 bytes, in that order.
    const int a_row0 = kRowsPerDma * G::kDmaA * wave;
    const int b_row0 = kRowsPerDma * G::kDmaB * wave;
    const uint32_t kblocks = (uint32_t)(K / kStageK);
    // scale DMA: 64 rows of one operand per instruction, 16 bytes (one group) per lane. The
    // tile's 64-row chunks (A's first, then B's) go round-robin over the wavefronts: instruction u
    // of wavefront w brings chunk (w + NW u) mod kScaleChunks. Where the chunks do not divide
    // evenly, the last wavefronts load a chunk a second time (the same bytes to the same place),
    // so that every wavefront issues the same number of loads and its vmcnt waits count alike.
    int s_dst[G::kDmaPerScales];
#pragma unroll
    for (int u = 0; u < G::kDmaPerScales; ++u) {
        const int chunk = (wave + NW * u) % G::kScaleChunks;
        const bool is_b = chunk >= TM / 64;
        s_dst[u] = (is_b ? TM * 16 : 0) + 1024 * (is_b ? chunk - TM / 64 : chunk);
    }
    // this lane's DMA sources for the tile at w
    using Offs = DmaOffsets<G::kDmaA, G::kDmaB, G::kDmaPerScales>;
    auto offsets_of = [&](const TileWhere &w) {
        Offs o;
#pragma unroll
        for (int u = 0; u < G::kDmaA; ++u) {
            if constexpr (TILED) {
                const uint32_t rb = (uint32_t)(w.m0 + a_row0 + kRowsPerDma * u) / 16;
                o.a[u] = rb * kblocks * 1024u + (uint32_t)lane * 16u;
            } else {
                const int row = a_row0 + kRowsPerDma * u + lane / 4;
                const int chunk = (lane % 4) ^ chunk_perm(row);
                o.a[u] = (uint32_t)(min(w.m0 + row, M - 1) * lda + 16 * chunk);
            }
        }
#pragma unroll
        for (int u = 0; u < G::kDmaB; ++u) {
            if constexpr (TILED) {
                const uint32_t rb = (uint32_t)(w.n0 + b_row0 + kRowsPerDma * u) / 16;
                o.b[u] = rb * kblocks * 1024u + (uint32_t)lane * 16u;
            } else {
                const int row = b_row0 + kRowsPerDma * u + lane / 4;
                const int chunk = (lane % 4) ^ chunk_perm(row);
                o.b[u] = (uint32_t)(min(w.n0 + row, N - 1) * ldb + 16 * chunk);
            }
        }
#pragma unroll
        for (int u = 0; u < G::kDmaPerScales; ++u) {
            const int chunk = (wave + NW * u) % G::kScaleChunks;
            const bool is_b = chunk >= TM / 64;
            const int q64 = is_b ? chunk - TM / 64 : chunk;
            const int row = 64 * q64 + lane;
            o.src[u] = is_b ? w.bs : w.as;
            if constexpr (TILED) {
                // 64-row x 512-K scale blocks of 1024 bytes, 16 per row
                o.s[u] = ((uint32_t)(is_b ? w.n0 : w.m0) / 64 + (uint32_t)q64) * ((uint32_t)K / 512) * 1024u +
                         (uint32_t)lane * 16u;
            } else {
                o.s[u] = (uint32_t)(is_b ? min(w.n0 + row, N - 1) * ldbs : min(w.m0 + row, M - 1) * ldas);
            }
        }
        return o;
    };
    Offs offs = offsets_of(cur);
    // fragment and scale reads of this lane
    const int perm = chunk_perm(r);
    const int a_frag = (wm * G::kWaveRows + r) * kRowBytes;
    const int b_frag = kABytes + (wn * G::kWaveCols + r) * kRowBytes;
    const int chunk0 = 16 * ((0 + half) ^ perm);
    const int chunk1 = 16 * ((2 + half) ^ perm);
    const int sa_lds = kScaleBase + 16 * (wm * G::kWaveRows + r);
    const int sb_lds = kScaleBase + 16 * (TM + wn * G::kWaveCols + r);

    const int stage0 = split * (K / kStageK / splits);  // first stage of this split
    // stage numbers past the tile's last one (nk + i) mean stage i of the next tile, once the
    // offsets have been set for it (the persistent walk)
    int shift = 0;
    auto dma = [&](int buf, int stage) {
        uint8_t *dst = lds + kRingBase + buf * kStageBytes;
        const uint32_t step = TILED ? 1024u : (uint32_t)kRowBytes;
        const uint8_t *asrc = aq + (uint32_t)(stage0 + stage - shift) * step;
        const uint8_t *bsrc = bq + (uint32_t)(stage0 + stage - shift) * step;
#pragma unroll
        for (int u = 0; u < G::kDmaA; ++u)
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(asrc + offs.a[u]),
                                             (lds_void_t *)(dst + a_row0 * kRowBytes + u * 1024), 16, 0, 0);
#pragma unroll
        for (int u = 0; u < G::kDmaB; ++u)
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(bsrc + offs.b[u]),
                                             (lds_void_t *)(dst + kABytes + b_row0 * kRowBytes + u * 1024), 16, 0,
                                             0);
    };
    auto dma_scales = [&](int g) {
        uint8_t *dst = lds + kScaleBase + (g & 1) * kScaleSlot;
#pragma unroll
        for (int u = 0; u < G::kDmaPerScales; ++u)
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(offs.src[u] + (TILED ? 1024u : 16u) *
                                                                         (uint32_t)(stage0 / 4 + g - shift / 4) +
                                                             offs.s[u]),
                                             (lds_void_t *)(dst + s_dst[u]), 16, 0, 0);
    };
    auto read_frags = [&](int buf, int chunk, u32x4 (&fa)[FI], u32x4 (&fb)[FJ]) {
        const uint8_t *src = lds + kRingBase + buf * kStageBytes;
#pragma unroll
        for (int i = 0; i < FI; ++i)
            fa[i] = *reinterpret_cast<const u32x4 *>(src + a_frag + 32 * i * kRowBytes + chunk);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            fb[j] = *reinterpret_cast<const u32x4 *>(src + b_frag + 32 * j * kRowBytes + chunk);
    };
    // this lane's scale words of stage s (byte 2 kk + half of word s % 4 of its rows)
    auto read_scales = [&](int s, uint32_t (&sa)[FI], uint32_t (&sb)[FJ]) {
        const int off = ((s >> 2) & 1) * kScaleSlot + 4 * (s & 3);
#pragma unroll
        for (int i = 0; i < FI; ++i)
            sa[i] = *reinterpret_cast<const uint32_t *>(lds + sa_lds + off + 16 * 32 * i);
#pragma unroll
        for (int j = 0; j < FJ; ++j)
            sb[j] = *reinterpret_cast<const uint32_t *>(lds + sb_lds + off + 16 * 32 * j);
    };

    v16f acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
        for (int j = 0; j < FJ; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // FI x FJ MFMAs of one 64-wide sub-step; transposed product: acc[i][j] holds C^T tile (j, i)
    auto mfma_step = [&](const u32x4 (&fa)[FI], const u32x4 (&fb)[FJ], const uint32_t (&sa)[FI],
                         const uint32_t (&sb)[FJ], auto opsel) {
        uint32_t xa[FI], xb[FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i) xa[i] = sa[i] >> (8 * half);
#pragma unroll
        for (int j = 0; j < FJ; ++j) xb[j] = sb[j] >> (8 * half);
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                mfma_t<decltype(opsel)::value>(acc[i][j], fb[j], fa[i], xb[j], xa[i]);
    };

    const int nk = K / kStageK / (PERSIST ? 1 : splits);  // stages of this split: a multiple of 4, >= 4
    const int ngroups = nk / 4;
    u32x4 fa0[FI], fb0[FJ], fa1[FI], fb1[FJ];
    uint32_t sa0[FI], sb0[FJ], sa1[FI], sb1[FJ];

    // prologue: scales of stages 0-3, then stages 0, 1, 2; wait for the scales and stage 0
    dma_scales(0);
    dma(0, 0);
    dma(1, 1);
    dma(2, 2);
    wait_vmcnt<2 * G::kDmaPerStage>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(0, chunk0, fa0, fb0);
    read_scales(0, sa0, sb0);

    constexpr int kMfma = FI * FJ;                 // MFMAs per sub-step
    constexpr int kFragReads = FI + FJ;

    // One stage s = 4 g + J (ring buffer J). WAITN = the number of loads issued after those of
    // stage s + 1 at the point of the wait (-1: no next stage); DMA_NEXT: issue stage s + 3;
    // SCALES_NEXT: issue the scales of group g + 1.
    auto stage = [&](int g, auto J, auto WAITN, auto DMA_NEXT, auto SCALES_NEXT) {
        constexpr int j = decltype(J)::value;
        constexpr int waitn = decltype(WAITN)::value;
        const int s = 4 * g + j;
        // sub-step 0: read sub-step 1's fragments while these MFMAs run, two after each of the
        // first MFMAs
        read_frags(j, chunk1, fa1, fb1);
        mfma_step(fa0, fb0, sa0, sb0, std::integral_constant<int, 0>());
        constexpr int lead0 = (kFragReads + 1) / 2;
#pragma unroll
        for (int k = 0; k < lead0; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfma - lead0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (waitn >= 0) {
            // stage s + 1 has landed for every wavefront, and every wavefront is done reading
            // stage s - 1's buffer, which the DMA of stage s + 3 overwrites
            wait_vmcnt<waitn>();
            __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(DMA_NEXT)::value) dma((j + 3) % 4, s + 3);
        if constexpr (decltype(SCALES_NEXT)::value) dma_scales(g + 1);
        if constexpr (waitn >= 0) {
            read_frags((j + 1) % 4, chunk0, fa0, fb0);
            read_scales(s + 1, sa1, sb1);
        }
        mfma_step(fa1, fb1, sa0, sb0, std::integral_constant<int, 2>());
        // the DMA first (it has the longest way to go), two instructions per MFMA, then the
        // next stage's fragment and scale reads, early enough to land before sub-step 0
        constexpr int nvmem = (decltype(DMA_NEXT)::value ? G::kDmaPerStage : 0) +
                              (decltype(SCALES_NEXT)::value ? G::kDmaPerScales : 0);
        constexpr int nds = waitn >= 0 ? kFragReads + (kFragReads + 1) / 2 : 0;
        constexpr int lv = (nvmem + 1) / 2, ld = (nds + 1) / 2;
        constexpr int lead1 = lv + ld < kMfma ? lv + ld : kMfma;
#pragma unroll
        for (int k = 0; k < lv; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // VMEM read (DMA)
        }
#pragma unroll
        for (int k = 0; k < ld; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMfma - lead1, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < FI; ++i) sa0[i] = sa1[i];
#pragma unroll
        for (int jj = 0; jj < FJ; ++jj) sb0[jj] = sb1[jj];
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using WS = std::integral_constant<int, G::kDmaPerStage>;
    using WSS = std::integral_constant<int, G::kDmaPerStage + G::kDmaPerScales>;
    using W0 = std::integral_constant<int, 0>;
    using WNone = std::integral_constant<int, -1>;
    using T = std::true_type;
    using F = std::false_type;

    // segmented accumulation: the sum of the finished segments, in K order
    v16f seg_sum[FOLD ? FI : 1][FOLD ? FJ : 1];
    if constexpr (FOLD) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) seg_sum[i][j] = v16f{};
    }

    // the epilogue of the tile at (m0, n0): acc[i][j] register q * 4 + t of lane (r, half) is
    // C[m0 + kWaveRows wm + 32 i + r][n0 + kWaveCols wn + 32 j + 8 q + 4 half + t]. With split-K
    // the unscaled partial product goes to partials[split][M][N] (FP32, beta 0) instead.
    auto epilogue = [&]() {
        // the lane index passes through an empty asm statement, so that the address arithmetic
        // below is formed per tile, after the main loop, instead of being hoisted out of the
        // persistent walk and held in registers through it
        int lane = tid & 63;
        if constexpr (PERSIST) asm volatile("" : "+v"(lane));
        const int r = lane & 31, half = lane >> 5;
        if (!PERSIST && splits > 1) out = OutSpec{partials + (int64_t)split * M * N, N, 1.0f, 0.0f, 0};
        float *c = static_cast<float *>(out.c);
        const int64_t ldc = out.ldc;
        const float alpha = out.alpha;
        // split-K partials are FP32 whatever the variant: a bf16 variant decides per launch
        const bool bf16_now = EPI == kEpiBF16 && out.bf16;
        const bool full_cols = n0 + TN <= N && (bf16_now ? out_vector_ok<true>(out) : out_vector_ok<false>(out));
        if (full_cols) {
            // stage each 32-row slice of this wavefront's kWaveRows x kWaveCols result through LDS
            // so that a store instruction writes whole rows (64 / (kWaveCols / 4) rows of kWaveCols
            // floats). Rows are padded by 16 bytes against bank conflicts; in the persistent walk
            // they are unpadded, their 16-byte chunks XOR-permuted by the row instead.
            constexpr int kEpiRow = G::kWaveCols * 4 + (PERSIST ? 0 : 16);   // bytes per staged row
            constexpr int kEpiWave = 32 * kEpiRow;                         // one slice per wavefront
            constexpr int kLanesPerRow = G::kWaveCols / 4;                 // 16-byte pieces per row
            constexpr int kRowsPerStore = 64 / kLanesPerRow;
            static_assert(!PERSIST || kLanesPerRow >= 16, "the chunk permutation spans 16 chunks");
            const auto at = [](int row, int col_bytes) {
                return PERSIST ? row * kEpiRow + ((col_bytes >> 4) ^ (row & 15)) * 16 : row * kEpiRow + col_bytes;
            };
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();                    // every wavefront is done with the stages
            __builtin_amdgcn_sched_barrier(0);
            uint8_t *epi = lds + (PERSIST ? kSliceOut : 0) + wave * kEpiWave;
#pragma unroll
            for (int i = 0; i < FI; ++i) {
#pragma unroll
                for (int jj = 0; jj < FJ; ++jj)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x4v v = {acc[i][jj][4 * q + 0], acc[i][jj][4 * q + 1], acc[i][jj][4 * q + 2],
                                          acc[i][jj][4 * q + 3]};
                        *reinterpret_cast<f32x4v *>(epi + at(r, (32 * jj + 8 * q + 4 * half) * 4)) = v;
                    }
                constexpr int kStores = 32 / kRowsPerStore;
                const int cc = 4 * (lane % kLanesPerRow);
                const int64_t ncol = n0 + wn * G::kWaveCols + cc;
                if constexpr (EPI == kEpiF32) {
#pragma unroll
                    for (int p = 0; p < kStores; ++p) {
                        const int rr = kRowsPerStore * p + lane / kLanesPerRow;
                        f32x4v v = *reinterpret_cast<const f32x4v *>(epi + at(rr, cc * 4));
                        v = v * alpha;
                        const int m = m0 + wm * G::kWaveRows + 32 * i + rr;
                        if (m < M) *reinterpret_cast<f32x4v *>(c + (int64_t)m * ldc + ncol) = v;
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < kStores; ++p) {
                        const int rr = kRowsPerStore * p + lane / kLanesPerRow;
                        f32x4v v = *reinterpret_cast<const f32x4v *>(epi + at(rr, cc * 4));
                        v = v * alpha;
                        const int m = m0 + wm * G::kWaveRows + 32 * i + rr;
                        if (m < M) {
                            if (bf16_now)
                                store4<true>(out, m, ncol, N, v, true);
                            else
                                store4<false>(out, m, ncol, N, v, true);
                        }
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int m = m0 + wm * G::kWaveRows + 32 * i + r;
            if (m >= M) continue;
            float *crow = c + (int64_t)m * ldc;
#pragma unroll
            for (int jj = 0; jj < FJ; ++jj)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * G::kWaveCols + 32 * jj + 8 * q + 4 * half;
                    const f32x4v v = {alpha * acc[i][jj][4 * q + 0], alpha * acc[i][jj][4 * q + 1],
                                      alpha * acc[i][jj][4 * q + 2], alpha * acc[i][jj][4 * q + 3]};
                    if constexpr (EPI == kEpiBF16) {
                        if (bf16_now)
                            store4<true>(out, m, n, N, v, false);
                        else
                            store4<false>(out, m, n, N, v, false);
                    } else if constexpr (EPI == kEpiF32Beta) {
                        store4<false>(out, m, n, N, v, false);
                    } else if (full_cols) {
                        *reinterpret_cast<f32x4v *>(crow + n) = v;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < N) crow[n + e] = v[e];
                    }
                }
        }
    };

    // virtual blocks of the launch (the persistent walk's range)
    const int nblocks = GROUP ? total * grp.count : total * splits;
    for (;;) {
        // the next tile of the walk (after the last one: this tile again), located now, while the
        // registers of the last stages are not yet needed
        bool has_next = false;
        TileWhere next{};
        Offs next_offs{};
        if constexpr (PERSIST) {
            has_next = vblock + (int)gridDim.x < nblocks;
            next = locate(has_next ? vblock + (int)gridDim.x : vblock);
            next_offs = offsets_of(next);
            // formed here (empty asm statements): left to the scheduler, the arithmetic sinks into
            // the last stages, where the fragments already hold most registers
#pragma unroll
            for (int u = 0; u < G::kDmaA; ++u) asm volatile("" : "+v"(next_offs.a[u]));
#pragma unroll
            for (int u = 0; u < G::kDmaB; ++u) asm volatile("" : "+v"(next_offs.b[u]));
#pragma unroll
            for (int u = 0; u < G::kDmaPerScales; ++u) asm volatile("" : "+v"(next_offs.s[u]));
        }
        for (int g = 0; g + 1 < ngroups; ++g) {
            stage(g, I0(), WS(), T(), T());
            stage(g, I1(), WSS(), T(), F());
            stage(g, I2(), WSS(), T(), F());
            stage(g, I3(), WS(), T(), F());
            if constexpr (FOLD) {
                if ((g + 1) % fold_groups == 0) {
#pragma unroll
                    for (int i = 0; i < FI; ++i)
#pragma unroll
                        for (int j = 0; j < FJ; ++j) {
                            seg_sum[i][j] = seg_sum[i][j] + acc[i][j];
                            acc[i][j] = v16f{};
                        }
                }
            }
        }
        const int g = ngroups - 1;
        if constexpr (PERSIST) {
            stage(g, I0(), WS(), T(), F());
            // every load of this tile is issued: the DMA now brings the next tile's stages 0 and 1
            // (as stages nk and nk + 1, into ring buffers 0 and 1) and its group-0 scales (slot 0,
            // free since the number of groups is even). After the last tile the same loads bring
            // this tile's first stages again, unused, so that one code path serves both.
            offs = next_offs;
            aq = next.aq;
            bq = next.bq;
            shift = nk;
            stage(g, I1(), WS(), T(), T());
            stage(g, I2(), WSS(), T(), F());
            stage(g, I3(), WNone(), F(), F());
        } else {
            stage(g, I0(), WS(), T(), F());
            stage(g, I1(), WS(), F(), F());
            stage(g, I2(), W0(), F(), F());
            stage(g, I3(), WNone(), F(), F());
        }
        if constexpr (FOLD) {
            // the last segment joins the earlier ones
#pragma unroll
            for (int i = 0; i < FI; ++i)
#pragma unroll
                for (int j = 0; j < FJ; ++j) acc[i][j] = seg_sum[i][j] + acc[i][j];
        }
        // the walk: the next tile's first stages and scales land before any store is issued, so
        // that nothing waits for the stores to drain until the next tile's first stage
        if constexpr (PERSIST) wait_vmcnt<0>();
        epilogue();
        if (!has_next) return;

        // the next tile: its stages 0 and 1 and scales landed before this wavefront's first store
        // (vmcnt 0 above), every wavefront's once all have passed the barrier, which also ends the
        // staged epilogue's reads of ring buffers 2 and 3. The stores drain meanwhile: the first
        // stage's wait counts them too.
        vblock += (int)gridDim.x;
        split = next.split;
        m0 = next.m0;
        n0 = next.n0;
        out.c = next.c;
        shift = 0;
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                acc[i][j] = v16f{};
                if constexpr (FOLD) seg_sum[i][j] = v16f{};
            }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        dma(2, 2);
        read_frags(0, chunk0, fa0, fb0);
        read_scales(0, sa0, sb0);
    }
}

// an empty contraction: c = beta * c (c = 0 when beta is 0, without reading c)
__global__ __launch_bounds__(256) void empty_product_kernel(OutSpec out, int64_t M, int64_t N)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < M * N) store1_any(out, i / N, i % N, 0.0f);
}

// c[m][n] = alpha * (p_0[m][n] + p_1[m][n] + ... + p_{S-1}[m][n]) (+ beta * c), summed in that
// fixed order
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ p, int splits, int64_t M,
                                                            int64_t N, OutSpec out)
{
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N) return;
    const int64_t mn = M * N;
    float acc = p[i];
    for (int s = 1; s < splits; ++s) acc += p[(int64_t)s * mn + i];
    store1_any(out, i / N, i % N, out.alpha * acc);
}

}  // namespace

hipError_t launch_empty_product(void *c, bool bf16, int64_t M, int64_t N, int64_t ldc, float beta,
                                hipStream_t stream)
{
    const int64_t total = M * N;
    if (total == 0) return hipSuccess;
    return launch(empty_product_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                  OutSpec{c, ldc, 0.0f, beta, bf16 ? 1 : 0}, M, N);
}

int gemm_splits(int64_t M, int64_t N, int64_t K)
{
    // split the contraction only when the output has at most 32 tiles of 256 x 256 (an eighth of
    // the compute units): under the board's power cap a few busy CUs clock higher, and at 64
    // tiles the partials' extra HBM traffic already cancels the gain. Each split keeps at least
    // 1024 values of K (whole 512-groups).
    const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
    if (K % 512 != 0 || tiles > 32) return 1;
    int s = 1;
    while (s < 8 && tiles * s * 2 <= 256 && (K / 512) % (s * 2) == 0 && K / (512 * s * 2) >= 2) s *= 2;
    // each split's chain (one rounding per 32 K) plus the fixed-order sum of the partials must
    // stay within the rounding bound; otherwise one workgroup per tile with a segmented chain
    if (s > 1 && K / 32 / s + s > kMaxDepth) return 1;
    return s;
}

// the persistent walk (256 x 256 tiles, and the 256 x 128 tiles of segmented chains): more
// tiles than CUs, and an even number of 512-wide groups per contraction (the next tile's first
// scales go to the slot the last group leaves free)
static bool persistent_ok(int64_t tiles, int64_t K) { return tiles > kComputeUnits && K % 1024 == 0; }

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    const int s = gemm_splits(M, N, K);
    return s > 1 ? (size_t)s * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                       const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs, int64_t M,
                       int64_t N, int64_t K, float alpha, float beta, void *c, bool bf16, int64_t ldc,
                       bool tiled, void *workspace, size_t ws_bytes, hipStream_t stream)
{
    const OutSpec out{c, ldc, alpha, beta, bf16 ? 1 : 0};
    const int epi = bf16 ? kEpiBF16 : (beta != 0.0f ? kEpiF32Beta : kEpiF32);
    const int tiles_m = (int)((M + kBM - 1) / kBM), tiles_n = (int)((N + kBN - 1) / kBN);
    const bool scales_aligned = ((uintptr_t)as % 16 == 0) && ((uintptr_t)bs % 16 == 0) &&
                                ldas % 16 == 0 && ldbs % 16 == 0;
    const bool offsets_fit = (int64_t)(M - 1) * lda + lda <= INT32_MAX && (int64_t)(N - 1) * ldb + ldb <= INT32_MAX;
    // tiled: the caller guarantees K % 512 == 0 and buffers padded to whole 256-row tiles
    const bool pipelined = tiled || (K % 512 == 0 && K > 0 && scales_aligned && offsets_fit);
    if (!pipelined) {
        const dim3 sgrid((unsigned)((N + kTileN - 1) / kTileN), (unsigned)((M + kTileM - 1) / kTileM));
        // two blocks per 64-wide step
        const int fold_steps = chain_segment((K + 63) / 64, 2);
        if (fold_steps > 0)
            return launch(gemm_mxfp4_simple<true>, sgrid, dim3(256), 0, stream, aq, lda, as, ldas, bq, ldb, bs,
                          ldbs, (int)M, (int)N, (int)K, out, fold_steps, GroupArgs{});
        return launch(gemm_mxfp4_simple<false>, sgrid, dim3(256), 0, stream, aq, lda, as, ldas, bq, ldb, bs, ldbs,
                      (int)M, (int)N, (int)K, out, 0, GroupArgs{});
    }
    int splits = gemm_splits(M, N, K);
    if (splits > 1 && (workspace == nullptr || ws_bytes < gemm_workspace_bytes(M, N, K) ||
                       (uintptr_t)workspace % 16 != 0))
        splits = 1;
    float *partials = splits > 1 ? static_cast<float *>(workspace) : nullptr;
    // an unsplit contraction longer than one chain may be: segments of whole groups (16 blocks)
    const int fold = splits == 1 ? chain_segment(K / 512, 16) : 0;
    hipError_t e;
    // pick one kernel variant by layout and epilogue (FOLD: segmented accumulation)
    auto pick = [&](auto run_kernel, auto nw, auto tm, auto tn, auto wm, auto fold_v) {
        constexpr int NW = decltype(nw)::value, TM = decltype(tm)::value, TN = decltype(tn)::value;
        constexpr int WM = decltype(wm)::value;
        constexpr bool FOLD = decltype(fold_v)::value;
        if (tiled)
            return epi == kEpiBF16 ? run_kernel(gemm_mxfp4_pipelined<NW, true, kEpiBF16, TM, TN, WM, FOLD>)
                 : epi == kEpiF32Beta ? run_kernel(gemm_mxfp4_pipelined<NW, true, kEpiF32Beta, TM, TN, WM, FOLD>)
                                      : run_kernel(gemm_mxfp4_pipelined<NW, true, kEpiF32, TM, TN, WM, FOLD>);
        return epi == kEpiBF16 ? run_kernel(gemm_mxfp4_pipelined<NW, false, kEpiBF16, TM, TN, WM, FOLD>)
             : epi == kEpiF32Beta ? run_kernel(gemm_mxfp4_pipelined<NW, false, kEpiF32Beta, TM, TN, WM, FOLD>)
                                  : run_kernel(gemm_mxfp4_pipelined<NW, false, kEpiF32, TM, TN, WM, FOLD>);
    };
    using C4 = std::integral_constant<int, 4>;
    using C2 = std::integral_constant<int, 2>;
    using C128 = std::integral_constant<int, 128>;
    using C256 = std::integral_constant<int, 256>;
    if (splits == 1 && fold > 0 && tiles_m * tiles_n >= kComputeUnits / 2) {
        // segmented chains on a full grid (from 128 large tiles, i.e. 256 of these: one per CU,
        // measured 2-3% faster than 512 of 128 x 128 at 1024 x 4096 x 8192 and 4096 x 2048 x
        // 14336): the 256 x 128 tile
        const int mm = (int)((M + kFoldTM - 1) / kFoldTM), mn = (int)((N + kFoldTN - 1) / kFoldTN);
        if (epi == kEpiF32 && persistent_ok(mm * mn, K)) {
            const auto run_walk = [&](auto kernel) {
                return launch(kernel, dim3(kComputeUnits), dim3(64 * kFoldWaves), 0, stream, aq, lda, as, ldas, bq,
                              ldb, bs, ldbs, (int)M, (int)N, (int)K, out, mm, mn, 1, (float *)nullptr, fold,
                              GroupArgs{});
            };
            return tiled ? run_walk(gemm_mxfp4_pipelined<kFoldWaves, true, kEpiF32, kFoldTM, kFoldTN, 4, true, false,
                                                         true>)
                         : run_walk(gemm_mxfp4_pipelined<kFoldWaves, false, kEpiF32, kFoldTM, kFoldTN, 4, true, false,
                                                         true>);
        }
        const auto run_mid = [&](auto kernel) {
            return launch(kernel, dim3((unsigned)(mm * mn)), dim3(64 * kFoldWaves), 0, stream, aq, lda, as, ldas, bq,
                          ldb, bs, ldbs, (int)M, (int)N, (int)K, out, mm, mn, 1, (float *)nullptr, fold,
                          GroupArgs{});
        };
        return pick(run_mid, std::integral_constant<int, kFoldWaves>(), std::integral_constant<int, kFoldTM>(),
                    std::integral_constant<int, kFoldTN>(), C4(), std::true_type());
    }
    if (splits == 1 && (fold > 0 || tiles_m * tiles_n <= kComputeUnits / 2)) {
        // 256 x 256 tiles would leave at least half the compute units idle: 128 x 128 tiles, four
        // wavefronts, two workgroups per CU, four times as many workgroups. Measured faster up to
        // 128 large tiles (8192 x 1024 x 4096: 28.2 -> 24.6 us; 1024 x 4096 x 8192: 45.9 -> 24.0 us)
        // and slower from 192 on (8192 x 1536 x 4096: 33.0 -> 35.2 us), where the small tiles'
        // doubled operand traffic costs more than the extra workgroups gain.
        const int sm = (int)((M + 127) / 128), sn = (int)((N + 127) / 128);
        const auto run_small = [&](auto kernel) {
            return launch(kernel, dim3((unsigned)(sm * sn)), dim3(64 * 4), 0, stream, aq, lda, as, ldas, bq, ldb, bs,
                          ldbs, (int)M, (int)N, (int)K, out, sm, sn, 1, (float *)nullptr, fold, GroupArgs{});
        };
        if (fold > 0) return pick(run_small, C4(), C128(), C128(), C2(), std::true_type());
        return pick(run_small, C4(), C128(), C128(), C2(), std::false_type());
    }
    if (splits == 1 && epi == kEpiF32 && persistent_ok(tiles_m * tiles_n, K)) {
        // more tiles than CUs: one workgroup per CU walks them
        const auto run_walk = [&](auto kernel) {
            return launch(kernel, dim3(kComputeUnits), dim3(64 * kGemmWaves), 0, stream, aq, lda, as, ldas, bq, ldb,
                          bs, ldbs, (int)M, (int)N, (int)K, out, tiles_m, tiles_n, 1, (float *)nullptr, 0,
                          GroupArgs{});
        };
        return tiled ? run_walk(gemm_mxfp4_pipelined<kGemmWaves, true, kEpiF32, kBM, kBN, 2, false, false, true>)
                     : run_walk(gemm_mxfp4_pipelined<kGemmWaves, false, kEpiF32, kBM, kBN, 2, false, false, true>);
    }
    const dim3 grid((unsigned)(tiles_m * tiles_n * splits)), block(64 * kGemmWaves);
    const auto run = [&](auto kernel) {
        return launch(kernel, grid, block, 0, stream, aq, lda, as, ldas, bq, ldb, bs, ldbs, (int)M, (int)N, (int)K,
                      out, tiles_m, tiles_n, splits, partials, 0, GroupArgs{});
    };
    e = pick(run, std::integral_constant<int, kGemmWaves>(), C256(), C256(), C2(), std::false_type());
    if (e != hipSuccess || splits == 1) return e;
    const int64_t total = M * N;
    return launch(splitk_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                  (const float *)partials, splits, M, N, out);
}

hipError_t launch_gemm_grouped(const GemmGroupItem *items, int count, int64_t lda, int64_t ldas, int64_t ldb,
                               int64_t ldbs, int64_t M, int64_t N, int64_t K, float alpha, int64_t ldc, bool tiled,
                               hipStream_t stream)
{
    const bool scales_aligned = ldas % 16 == 0 && ldbs % 16 == 0;
    const bool offsets_fit = (int64_t)(M - 1) * lda + lda <= INT32_MAX && (int64_t)(N - 1) * ldb + ldb <= INT32_MAX;
    bool pipelined = tiled || (K % 512 == 0 && K > 0 && scales_aligned && offsets_fit);
    for (int i = 0; i < count; ++i)
        pipelined = pipelined && ((uintptr_t)items[i].as % 16 == 0) && ((uintptr_t)items[i].bs % 16 == 0);
    if (count > kGroupMax) {
        // product by product
        for (int i = 0; i < count; ++i) {
            const hipError_t e = launch_gemm(items[i].aq, lda, items[i].as, ldas, items[i].bq, ldb, items[i].bs,
                                             ldbs, M, N, K, alpha, 0.0f, items[i].c, false, ldc, tiled, nullptr, 0,
                                             stream);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    GroupArgs grp{};
    grp.count = count;
    for (int i = 0; i < count; ++i)
        grp.item[i] = GroupItem{items[i].aq, items[i].as, items[i].bq, items[i].bs, items[i].c};
    const OutSpec out{items[0].c, ldc, alpha, 0.0f, 0};
    if (!pipelined) {
        // the row kernel, one grid layer per product
        const dim3 sgrid((unsigned)((N + kTileN - 1) / kTileN), (unsigned)((M + kTileM - 1) / kTileM),
                         (unsigned)count);
        const int fold_steps = chain_segment((K + 63) / 64, 2);
        if (fold_steps > 0)
            return launch(gemm_mxfp4_simple<true>, sgrid, dim3(256), 0, stream, items[0].aq, lda, items[0].as, ldas,
                          items[0].bq, ldb, items[0].bs, ldbs, (int)M, (int)N, (int)K, out, fold_steps, grp);
        return launch(gemm_mxfp4_simple<false>, sgrid, dim3(256), 0, stream, items[0].aq, lda, items[0].as, ldas,
                      items[0].bq, ldb, items[0].bs, ldbs, (int)M, (int)N, (int)K, out, 0, grp);
    }
    const int fold = chain_segment(K / 512, 16);
    const int64_t big_tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN) * count;
    // the geometry launch_gemm would pick for one product with all the products' tiles
    auto run = [&](auto kernel, int nw, int tm, int tn) {
        const int gm = (int)((M + tm - 1) / tm), gn = (int)((N + tn - 1) / tn);
        return launch(kernel, dim3((unsigned)(gm * gn * count)), dim3(64 * nw), 0, stream, items[0].aq, lda,
                      items[0].as, ldas, items[0].bq, ldb, items[0].bs, ldbs, (int)M, (int)N, (int)K, out, gm, gn, 1,
                      (float *)nullptr, fold, grp);
    };
    // the walk over all the products' tiles of geometry tm x tn, one workgroup per CU
    auto run_walk = [&](auto kernel, int nw, int tm, int tn) {
        const int gm = (int)((M + tm - 1) / tm), gn = (int)((N + tn - 1) / tn);
        return launch(kernel, dim3(kComputeUnits), dim3(64 * nw), 0, stream, items[0].aq, lda, items[0].as, ldas,
                      items[0].bq, ldb, items[0].bs, ldbs, (int)M, (int)N, (int)K, out, gm, gn, 1, (float *)nullptr,
                      fold, grp);
    };
    if (fold > 0 && big_tiles >= kComputeUnits / 2) {   // as in launch_gemm
        const int64_t fold_tiles = ((M + kFoldTM - 1) / kFoldTM) * ((N + kFoldTN - 1) / kFoldTN) * count;
        if (persistent_ok(fold_tiles, K))
            return tiled ? run_walk(gemm_mxfp4_pipelined<kFoldWaves, true, kEpiF32, kFoldTM, kFoldTN, 4, true, true,
                                                         true>,
                                    kFoldWaves, kFoldTM, kFoldTN)
                         : run_walk(gemm_mxfp4_pipelined<kFoldWaves, false, kEpiF32, kFoldTM, kFoldTN, 4, true, true,
                                                         true>,
                                    kFoldWaves, kFoldTM, kFoldTN);
        return tiled ? run(gemm_mxfp4_pipelined<kFoldWaves, true, kEpiF32, kFoldTM, kFoldTN, 4, true, true>,
                           kFoldWaves, kFoldTM, kFoldTN)
                     : run(gemm_mxfp4_pipelined<kFoldWaves, false, kEpiF32, kFoldTM, kFoldTN, 4, true, true>,
                           kFoldWaves, kFoldTM, kFoldTN);
    }
    if (fold > 0)
        return tiled ? run(gemm_mxfp4_pipelined<4, true, kEpiF32, 128, 128, 2, true, true>, 4, 128, 128)
                     : run(gemm_mxfp4_pipelined<4, false, kEpiF32, 128, 128, 2, true, true>, 4, 128, 128);
    if (big_tiles <= kComputeUnits / 2)
        return tiled ? run(gemm_mxfp4_pipelined<4, true, kEpiF32, 128, 128, 2, false, true>, 4, 128, 128)
                     : run(gemm_mxfp4_pipelined<4, false, kEpiF32, 128, 128, 2, false, true>, 4, 128, 128);
    if (persistent_ok(big_tiles, K))
        return tiled ? run_walk(gemm_mxfp4_pipelined<kGemmWaves, true, kEpiF32, kBM, kBN, 2, false, true, true>,
                                kGemmWaves, kBM, kBN)
                     : run_walk(gemm_mxfp4_pipelined<kGemmWaves, false, kEpiF32, kBM, kBN, 2, false, true, true>,
                                kGemmWaves, kBM, kBN);
    return tiled ? run(gemm_mxfp4_pipelined<kGemmWaves, true, kEpiF32, kBM, kBN, 2, false, true>, kGemmWaves, kBM, kBN)
                 : run(gemm_mxfp4_pipelined<kGemmWaves, false, kEpiF32, kBM, kBN, 2, false, true>, kGemmWaves, kBM, kBN);
}

}  // namespace mx

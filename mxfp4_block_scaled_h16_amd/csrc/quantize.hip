// Fused rotate + amax + E8M0 scale + E2M1 encode + pack kernels (gfx950).
//
// The operand transform of the gist.science summary of "MXFP4 LLM pretraining", section 방법론
// (Methodology): deterministic block Hadamard (H16 / H32) along the GEMM's contraction axis, then
// MXFP4 quantization with nearest-even or stochastic rounding. Two kernels:
//   quant_rows -- along the contiguous axis (Fprop operands, the Dgrad gradient operand);
//   quant_cols -- along the strided axis, writing the quantized transpose (the Wgrad token axis,
//                 section "주요 기여 및 발견" §1: the weight gradient is where MXFP4 hurts most).
// Both are HBM-bound: 2 bytes read and 0.5 + 1/32 bytes written per bf16 element; nearest-even
// rounding uses the hardware FP4 conversion, stochastic rounding a Philox word per element.
#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------ quant_rows --
// A lane owns 8 consecutive elements (16 bytes of bf16, 32 of f32); lanes 4b .. 4b + 3 own one
// 32-element MX block, so every load instruction of a wavefront reads 64 consecutive 8-element
// groups. Hadamard stages of stride 1, 2, 4 run in registers, the stride-8 and stride-16
// stages across lanes l ^ 1 and l ^ 2; the block amax is reduced over the same quad. Each lane
// stores one 32-bit word of codes (consecutive lanes, consecutive words) and lane 4b the scale.
constexpr int kRowsUnroll = 4;  // 8-element groups per lane, 64 groups apart

template <bool F32>
__device__ __forceinline__ void load8(const char *p, float *v)
{
    if constexpr (F32) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p) + 1);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[2 * u] = bf16_lo(w[u]);
            v[2 * u + 1] = bf16_hi(w[u]);
        }
    }
}

// Tiled-layout byte offsets (see mxfp4.h): the 16-byte chunk of codes holding elements
// [32 c, 32 c + 32) of quantized row o, and the scale byte of that block.
__device__ __forceinline__ int64_t tiled_chunk(uint32_t o, uint32_t c, int64_t L)
{
    return ((int64_t)(o / 16) * (L / 128) + c / 4) * 1024 + (o % 16) * 64 + 16 * ((c % 4) ^ ((o % 16) / 4));
}
__device__ __forceinline__ int64_t tiled_scale(uint32_t o, uint32_t c, int64_t L)
{
    return ((int64_t)(o / 64) * (L / 512) + c / 16) * 1024 + (o % 64) * 16 + (c % 16);
}

template <int H, bool F32, bool SR, bool TILED>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t groups_per_row, uint32_t total_groups,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds, uint32_t key0,
    uint32_t key1, uint32_t stream_id, int64_t L)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t base = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * (64u * kRowsUnroll);
    const size_t esize = F32 ? 4 : 2;
    const bool upper1 = lane & 1, upper2 = lane & 2;

    float v[kRowsUnroll][8];
    uint32_t row[kRowsUnroll], grp[kRowsUnroll];
    bool live[kRowsUnroll];
    {
        // every lane runs (the cross-lane stages need the whole quad); a group past the end is
        // replaced by one of the last block, same lane within the quad, and is not stored
        uint32_t g = base + lane;
        live[0] = g < total_groups;
        if (!live[0]) g = total_groups - 4u + (lane & 3u);
        uint32_t r = g / groups_per_row;
        uint32_t c = g - r * groups_per_row;
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
            if (u > 0) {
                const uint32_t gu = base + 64u * u + lane;
                live[u] = gu < total_groups;
                if (live[u]) {
                    c += 64u;
                    while (c >= groups_per_row) {
                        c -= groups_per_row;
                        ++r;
                    }
                } else {
                    r = (total_groups - 4u) / groups_per_row;
                    c = total_groups - 4u + (lane & 3u) - r * groups_per_row;
                }
            }
            row[u] = r;
            grp[u] = c;
            load8<F32>(reinterpret_cast<const char *>(x) + ((int64_t)r * ldx + (int64_t)c * 8) * esize, v[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
        if constexpr (H >= 16) {
            fwht_regs<8>(v[u]);
            fwht_cross_stage<1>(v[u], upper1);
            if constexpr (H == 32) fwht_cross_stage<2>(v[u], upper2);
        }
        uint32_t amax = 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = max(amax, abs_bits(v[u][i]));
        amax = max(amax, quad_xor<1>(amax));
        amax = max(amax, quad_xor<2>(amax));
        const uint32_t sc = e8m0_from_amax_bits(amax);
        uint32_t word;
        if constexpr (SR) {
            const uint64_t index0 = (uint64_t)row[u] * (uint64_t)L + (uint64_t)grp[u] * 8u;
            word = encode8_stochastic(v[u], sc, index0, key0, key1, stream_id);
        } else {
            prescale_if_zero_scale<8>(v[u], sc);
            word = encode8_nearest(v[u], e8m0_divisor(sc));
        }
        if (sc == 0xFFu) word = 0u;
        if (live[u]) {
            if constexpr (TILED) {
                const int64_t at = tiled_chunk(row[u], grp[u] / 4, L) + 4 * (grp[u] % 4);
                __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(q + at));
                if ((lane & 3u) == 0u) scales[tiled_scale(row[u], grp[u] / 4, L)] = (uint8_t)sc;
            } else {
                __builtin_nontemporal_store(word, reinterpret_cast<uint32_t *>(q + (int64_t)row[u] * ldq) + grp[u]);
                if ((lane & 3u) == 0u) scales[(int64_t)row[u] * lds + grp[u] / 4] = (uint8_t)sc;
            }
        }
    }
}

// ------------------------------------------------------------------------------ quant_cols --
// Quantize along the strided axis and write the quantized transpose. A workgroup takes a tile of
// 256 rows (eight 32-row MX blocks) by 128 bytes of columns (64 bf16 / 32 f32):
//  1. each load instruction reads 8 rows x 128 bytes (row i of each of the eight blocks), stored
//     to LDS at row (i * 8 + block) so the instruction writes 1 KB contiguously;
//  2. a thread takes one block of one (f32) or two (bf16) columns, reads its 32 values with
//     ds_read_b32 (the two blocks of a wavefront sit in adjacent 128-byte LDS rows, so all 64
//     lanes hit distinct banks), rotates, scales and encodes in registers and puts 16 bytes of
//     codes per column into an LDS output tile;
//  3. the output tile goes out as whole 128-byte lines: quantized row = tile column, 8 blocks
//     x 16 bytes.
constexpr int kColsTileRows = 256;
constexpr int kColsRowBytes = 128;
constexpr int kColsOutStride = 144;  // 128 bytes of codes + 16 of padding per output row

template <int H, bool F32, bool SR, bool TILED>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t rows, uint32_t cols, uint32_t col_tiles,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds, uint32_t key0,
    uint32_t key1, uint32_t stream_id)
{
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kTileCols = kColsRowBytes / kEsize;   // 32 f32 or 64 bf16 columns
    constexpr int kColsPerThread = F32 ? 1 : 2;
    constexpr int kPerChunk = 16 / kEsize;              // elements per 16-byte chunk
    __shared__ __attribute__((aligned(16))) uint8_t tile[kColsTileRows * kColsRowBytes];
    __shared__ __attribute__((aligned(16))) uint8_t out[kTileCols * kColsOutStride];
    __shared__ uint8_t out_scales[kTileCols * 8];

    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t c0 = (blockIdx.x % col_tiles) * kTileCols;
    const uint32_t r0 = (blockIdx.x / col_tiles) * kColsTileRows;
    const uint32_t nblocks = min(8u, (rows - r0) / 32u);
    const char *xb = reinterpret_cast<const char *>(x);

    // 1. load: wavefront w brings rows i = 8 w .. 8 w + 7 of every block
    {
        const uint32_t blk = lane / 8, chunk = lane % 8;
        const uint32_t col = c0 + chunk * kPerChunk;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const uint32_t i = 8 * wave + k;
            u32x4 t = {0u, 0u, 0u, 0u};
            if (blk < nblocks) {
                const char *src = xb + ((int64_t)(r0 + 32 * blk + i) * ldx + col) * kEsize;
                if (col + kPerChunk <= cols) {
                    t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(src));
                } else {
                    // right edge: only the columns that exist
                    uint32_t e[4] = {0u, 0u, 0u, 0u};
                    for (int j = 0; j < kPerChunk && col + j < cols; ++j) {
                        uint32_t bits;
                        if constexpr (F32) bits = *reinterpret_cast<const uint32_t *>(src + 4 * j);
                        else bits = *reinterpret_cast<const uint16_t *>(src + 2 * j);
                        e[(j * kEsize) / 4] |= bits << (8 * ((j * kEsize) % 4));
                    }
                    t = u32x4{e[0], e[1], e[2], e[3]};
                }
            }
            *reinterpret_cast<u32x4 *>(tile + (i * 8 + blk) * kColsRowBytes + chunk * 16) = t;
        }
    }
    __syncthreads();

    // 2. one block of kColsPerThread columns per thread
    {
        const uint32_t cp = lane % 32, blk = 2 * wave + lane / 32;
        if (blk < nblocks) {
            float v[kColsPerThread][32];
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(tile + (i * 8 + blk) * kColsRowBytes + cp * 4);
                if constexpr (F32) {
                    v[0][i] = __uint_as_float(w);
                } else {
                    v[0][i] = bf16_lo(w);
                    v[1][i] = bf16_hi(w);
                }
            }
#pragma unroll
            for (int cc = 0; cc < kColsPerThread; ++cc) {
                const uint32_t tc = cp * kColsPerThread + cc;  // tile column = quantized row
                rotate_block<H>(v[cc]);
                uint32_t amax = 0u;
#pragma unroll
                for (int i = 0; i < 32; ++i) amax = max(amax, abs_bits(v[cc][i]));
                const uint32_t sc = e8m0_from_amax_bits(amax);
                uint32_t words[4];
                if constexpr (SR) {
                    const uint64_t index0 = (uint64_t)(c0 + tc) * (uint64_t)rows + (uint64_t)(r0 + 32 * blk);
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd)
                        words[wd] = encode8_stochastic(v[cc] + 8 * wd, sc, index0 + 8 * wd, key0, key1, stream_id);
                } else {
                    prescale_if_zero_scale<32>(v[cc], sc);
                    const float div = e8m0_divisor(sc);
#pragma unroll
                    for (int wd = 0; wd < 4; ++wd) words[wd] = encode8_nearest(v[cc] + 8 * wd, div);
                }
                if (sc == 0xFFu) words[0] = words[1] = words[2] = words[3] = 0u;
                *reinterpret_cast<u32x4 *>(out + tc * kColsOutStride + blk * 16) =
                    u32x4{words[0], words[1], words[2], words[3]};
                out_scales[tc * 8 + blk] = (uint8_t)sc;
            }
        }
    }
    __syncthreads();

    // 3. store: 8 lanes per quantized row, 16 bytes each (block = lane % 8)
#pragma unroll
    for (int pass = 0; pass < kTileCols / 32; ++pass) {
        const uint32_t tc = pass * 32 + tid / 8, blk = tid % 8;
        const uint32_t orow = c0 + tc;
        if (orow < cols && blk < nblocks) {
            const u32x4 t = *reinterpret_cast<const u32x4 *>(out + tc * kColsOutStride + blk * 16);
            const uint32_t kb = r0 / 32 + blk;  // block index along the quantized axis
            if constexpr (TILED) {
                __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(q + tiled_chunk(orow, kb, rows)));
                scales[tiled_scale(orow, kb, rows)] = out_scales[tc * 8 + blk];
            } else {
                __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(q + (int64_t)orow * ldq + kb * 16));
                scales[(int64_t)orow * lds + kb] = out_scales[tc * 8 + blk];
            }
        }
    }
}

template <int H, bool F32, bool SR, bool TILED>
hipError_t rows_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         hipStream_t stream)
{
    const uint32_t gpr = (uint32_t)(cols / 8);
    const uint32_t total = (uint32_t)(rows * (cols / 8));
    const uint32_t per_block = kThreads * kRowsUnroll;
    const dim3 grid((total + per_block - 1) / per_block);
    return launch(quant_rows_kernel<H, F32, SR, TILED>, grid, dim3(kThreads), 0, stream, x, ldx, gpr, total, q,
                  ldq, scales, lds, (uint32_t)seed, (uint32_t)(seed >> 32), stream_id, cols);
}

template <int H, bool F32, bool SR, bool TILED>
hipError_t cols_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         hipStream_t stream)
{
    const int64_t tile_cols = kColsRowBytes / (F32 ? 4 : 2);
    const int64_t col_tiles = (cols + tile_cols - 1) / tile_cols;
    const int64_t row_tiles = (rows + kColsTileRows - 1) / kColsTileRows;
    return launch(quant_cols_kernel<H, F32, SR, TILED>, dim3((unsigned)(col_tiles * row_tiles)), dim3(kThreads), 0,
                  stream, x, ldx, (uint32_t)rows, (uint32_t)cols, (uint32_t)col_tiles, q, ldq, scales, lds,
                  (uint32_t)seed, (uint32_t)(seed >> 32), stream_id);
}

template <template <int, bool, bool> class Sel, typename... A>
hipError_t pick(int h, bool f32, bool sr, A... a)
{
    // expands the 3 x 2 x 2 kernel variants
#define MX_CASE(HH)                                                                            \
    if (h == HH) {                                                                             \
        if (f32) return sr ? Sel<HH, true, true>::run(a...) : Sel<HH, true, false>::run(a...); \
        return sr ? Sel<HH, false, true>::run(a...) : Sel<HH, false, false>::run(a...);        \
    }
    MX_CASE(0)
    MX_CASE(16)
    MX_CASE(32)
#undef MX_CASE
    return hipErrorInvalidValue;
}

template <int H, bool F32, bool SR>
struct RowsSel {
    template <typename... A>
    static hipError_t run(bool tiled, A... a)
    {
        return tiled ? rows_dispatch<H, F32, SR, true>(a...) : rows_dispatch<H, F32, SR, false>(a...);
    }
};

template <int H, bool F32, bool SR>
struct ColsSel {
    template <typename... A>
    static hipError_t run(bool tiled, A... a)
    {
        return tiled ? cols_dispatch<H, F32, SR, true>(a...) : cols_dispatch<H, F32, SR, false>(a...);
    }
};

}  // namespace

hipError_t launch_quantize_rows(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<RowsSel>(hadamard, f32, stochastic, tiled, x, rows, cols, ldx, seed, stream_id, q, ldq,
                         scales, lds, stream);
}

hipError_t launch_quantize_cols(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<ColsSel>(hadamard, f32, stochastic, tiled, x, rows, cols, ldx, seed, stream_id, q, ldq,
                         scales, lds, stream);
}

}  // namespace mx

// Fused rotate + amax + E8M0 scale + E2M1 encode + pack kernels (gfx950).
//
// The operand transform of the gist.science summary of "MXFP4 LLM pretraining", section 방법론
// (Methodology): deterministic block Hadamard (H16 / H32) along the GEMM's contraction axis, then
// MXFP4 quantization with nearest-even or stochastic rounding. Three kernels:
//   quant_rows -- along the contiguous axis (Fprop operands, the Dgrad gradient operand);
//   quant_cols -- along the strided axis, writing the quantized transpose (the Wgrad token axis,
//                 section "주요 기여 및 발견" §1: the weight gradient is where MXFP4 hurts most);
//   quant_dual -- both from one read of the tensor, for up to 8 tensors per launch.
// Their bound is HBM: 2 bytes read and 0.5 + 1/32 bytes written per bf16 element (both axes:
// 2 + 2 x (0.5 + 1/32)); nearest-even rounding uses the hardware FP4 conversion, stochastic
// rounding a Philox word per element, whose 64-bit multiply-adds make those launches partly
// VALU-bound.
#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

// ------------------------------------------------------------------------------ quant_rows --
// A lane owns 16 consecutive elements (32 bytes of bf16, 64 of f32); lanes 2b, 2b + 1 own one
// 32-element MX block, so a wavefront covers 64 consecutive 16-element groups. H16 runs entirely
// in registers; H32's stride-16 stage crosses to lane l ^ 1, and so does the block amax. Each
// lane stores 8 bytes of codes (consecutive lanes, consecutive bytes) and lane 2b the scale.
// bf16 loads stay fully coalesced: each of a wavefront's two 16-byte loads reads 64 consecutive
// 8-element halves (lane l the half l / 32 of groups l % 32 and 32 + l % 32), and one
// v_permlane32_swap per register then hands every lane both halves of its own group.
constexpr int kRowsUnroll = 2;  // 16-element groups per lane, 64 groups apart

// 16 consecutive f32 values (f32 input keeps one lane's 64 bytes in four 16-byte loads)
__device__ __forceinline__ void load16_f32(const char *p, float *v)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 16 * k));
        v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
    }
}

// (lo, hi) -> lanes 0-31 keep lo and take the lo of lanes 32-63; lanes 32-63 take the hi of
// lanes 0-31 and keep hi: with lo = half h of group l % 32 and hi = half h of group 32 + l % 32
// (h = l / 32), lane l ends with both halves of group l.
__device__ __forceinline__ void pair_halves(u32x4 &lo, u32x4 &hi)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(lo[d], hi[d], false, false);
        lo[d] = r[0];
        hi[d] = r[1];
    }
}

__device__ __forceinline__ void unpack_bf16x16(const u32x4 &a, const u32x4 &b, float *v)
{
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        v[2 * u] = bf16_lo(w[u]);
        v[2 * u + 1] = bf16_hi(w[u]);
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

template <int H, bool F32, bool SR, bool TILED, bool RHT>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t groups_per_row, uint32_t total_groups,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds, uint32_t key0,
    uint32_t key1, uint32_t stream_id, int64_t L, uint32_t noclip, float norm, uint32_t last_row)
{
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t base = (blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)) * (64u * kRowsUnroll);
    const size_t esize = F32 ? 4 : 2;
    const bool upper1 = lane & 1;

    float v[kRowsUnroll][16];
    uint32_t row[kRowsUnroll], grp[kRowsUnroll];
    bool live[kRowsUnroll];
    if constexpr (!F32) {
        // groups base + 64 u + (lane % 32) (A) and + 32 (B): their halves lane / 32 are loaded,
        // then paired; a group past the end loads the last group instead and is not stored
        const uint32_t half = lane >> 5, ml = lane & 31u;
        uint32_t rA = (base + ml) / groups_per_row;
        uint32_t cA = base + ml - rA * groups_per_row;
        u32x4 lo[kRowsUnroll], hi[kRowsUnroll];
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
            if (u > 0) {
                cA += 64u;
                while (cA >= groups_per_row) {
                    cA -= groups_per_row;
                    ++rA;
                }
            }
            uint32_t rB = rA, cB = cA + 32u;
            while (cB >= groups_per_row) {
                cB -= groups_per_row;
                ++rB;
            }
            const uint32_t gA = base + 64u * u + ml;
            const bool liveA = gA < total_groups, liveB = gA + 32u < total_groups;
            live[u] = half ? liveB : liveA;
            row[u] = half ? rB : rA;
            grp[u] = half ? cB : cA;
            const uint32_t lrA = liveA ? rA : last_row, lcA = liveA ? cA : groups_per_row - 1u;
            const uint32_t lrB = liveB ? rB : last_row, lcB = liveB ? cB : groups_per_row - 1u;
            const uint16_t *xh = reinterpret_cast<const uint16_t *>(x);
            const u32x4 *pa = reinterpret_cast<const u32x4 *>(xh + (int64_t)lrA * ldx + (int64_t)lcA * 16 + 8 * half);
            const u32x4 *pb = reinterpret_cast<const u32x4 *>(xh + (int64_t)lrB * ldx + (int64_t)lcB * 16 + 8 * half);
            lo[u] = __builtin_nontemporal_load(pa);
            hi[u] = __builtin_nontemporal_load(pb);
        }
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u) {
            pair_halves(lo[u], hi[u]);
            unpack_bf16x16(lo[u], hi[u], v[u]);
        }
    } else {
        // every lane runs (the cross-lane steps need both lanes of a block); a group past the end
        // is replaced by one of the last block, same lane within the pair, and is not stored
        uint32_t g = base + lane;
        live[0] = g < total_groups;
        if (!live[0]) g = total_groups - 2u + (lane & 1u);
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
                    r = (total_groups - 2u) / groups_per_row;
                    c = total_groups - 2u + (lane & 1u) - r * groups_per_row;
                }
            }
            row[u] = r;
            grp[u] = c;
        }
        // all loads in flight before any is consumed
#pragma unroll
        for (int u = 0; u < kRowsUnroll; ++u)
            load16_f32(reinterpret_cast<const char *>(x) + ((int64_t)row[u] * ldx + (int64_t)grp[u] * 16) * esize, v[u]);
    }
#pragma unroll
    for (int u = 0; u < kRowsUnroll; ++u) {
        if constexpr (RHT) apply_signs<16>(v[u], (rht_sign_word(grp[u] / 2, key0, key1) >> (16 * (grp[u] % 2))) & 0xFFFFu);
        uint32_t amax;
        if constexpr (H == 16) {
            amax = fwht_regs_amax<16>(v[u]);
            if (norm != 1.0f) {
                scale_values<16>(v[u], norm);
                amax = scaled_amax(amax, norm);
            }
        } else {
            if constexpr (H == 32) {
                fwht_regs<16>(v[u]);
                fwht_cross_stage<1, 16>(v[u], upper1);
                if (norm != 1.0f) scale_values<16>(v[u], norm);
            }
            amax = amax_bits<16>(v[u]);
        }
        amax = max(amax, quad_xor<1>(amax));
        uint32_t sc = e8m0_from_amax_bits(amax);
        if (noclip) sc = e8m0_noclip(amax, sc);
        uint32_t w0, w1;
        prescale_if_zero_scale<16>(v[u], sc);
        const float div = e8m0_divisor(sc);
        if constexpr (SR) {
            const uint64_t index0 = (uint64_t)row[u] * (uint64_t)L + (uint64_t)grp[u] * 16u;
            uint32_t w[2];
            encode_stochastic<2>(v[u], div, index0, key0, key1, stream_id, w);
            w0 = w[0];
            w1 = w[1];
        } else {
            w0 = encode8_nearest(v[u], div);
            w1 = encode8_nearest(v[u] + 8, div);
        }
        if (sc == 0xFFu) w0 = w1 = 0u;
        const u32x2 codes = {w0, w1};
        if (live[u]) {
            if constexpr (TILED) {
                const int64_t at = tiled_chunk(row[u], grp[u] / 2, L) + 8 * (grp[u] % 2);
                __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(q + at));
                if ((lane & 1u) == 0u) scales[tiled_scale(row[u], grp[u] / 2, L)] = (uint8_t)sc;
            } else {
                __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(q + (int64_t)row[u] * ldq) + grp[u]);
                if ((lane & 1u) == 0u) scales[(int64_t)row[u] * lds + grp[u] / 2] = (uint8_t)sc;
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

template <int H, bool F32, bool SR, bool TILED, bool RHT>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t rows, uint32_t cols, uint32_t col_tiles,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds, uint32_t key0,
    uint32_t key1, uint32_t stream_id, uint32_t noclip, float norm)
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
            const uint32_t signs = RHT ? rht_sign_word(r0 / 32 + blk, key0, key1) : 0u;
#pragma unroll
            for (int cc = 0; cc < kColsPerThread; ++cc) {
                const uint32_t tc = cp * kColsPerThread + cc;  // tile column = quantized row
                if constexpr (RHT) apply_signs<32>(v[cc], signs);
                uint32_t amax = rotate_block_amax<H>(v[cc]);
                if (H > 0 && norm != 1.0f) {
                    scale_values<32>(v[cc], norm);
                    amax = scaled_amax(amax, norm);
                }
                uint32_t sc = e8m0_from_amax_bits(amax);
                if (noclip) sc = e8m0_noclip(amax, sc);
                uint32_t words[4];
                prescale_if_zero_scale<32>(v[cc], sc);
                const float div = e8m0_divisor(sc);
                if constexpr (SR) {
                    const uint64_t index0 = (uint64_t)(c0 + tc) * (uint64_t)rows + (uint64_t)(r0 + 32 * blk);
                    encode_stochastic<4>(v[cc], div, index0, key0, key1, stream_id, words);
                } else {
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

// ------------------------------------------------------------------------------ quant_dual --
// Both quantizations of one tensor from a single read of it: along each row (axis 1) and along
// each column (axis 0, written as the quantized transpose). Across Fprop, Dgrad and Wgrad each of
// X, W and dY is a contraction operand along both of its axes, so a training step needs both.
// A workgroup takes a 128 x 128-element tile:
//  1. a lane loads 16 consecutive elements of a row (8 lanes per row, 8 rows per wavefront
//     load), keeps the raw bits in an LDS tile and quantizes them along the row as quant_rows
//     does (Hadamard in registers, H32's last stage and the block amax across the lane pair,
//     8 bytes of codes per lane);
//  2. after a barrier a lane reads one column of one 32-row block (wavefront w: block w % 4,
//     column half w / 4; the 64 lanes read 64 consecutive elements of a row), rotates, scales
//     and encodes it as quant_cols does; after a barrier (every lane holds its column) the codes
//     go into the front of the same LDS tile, in the output's byte order, so that a workgroup
//     needs only the 32 KB tile (64 KB for f32);
//  3. after a second barrier the column output leaves as whole 1 KB tiled blocks (or as 16-byte
//     pieces of 64-byte row segments in the rows layout).
// Per bf16 element: 2 bytes read once, 2 x (0.5 + 1/32) bytes written.
constexpr int kDualTile = 128;
// Eight wavefronts per tile: a lane then quantizes two row groups and one column, half the
// serial work of four wavefronts. Measured faster at every size of the Llama-3.1-8B layer
// (the step's 18 dual launches 753 -> 716 us; 1024 x 4096 weights 9.0 -> 7.6 us).
constexpr int kDualWaves = 8;

struct DualOut {
    uint8_t *q;
    int64_t ldq;
    uint8_t *scales;
    int64_t lds;
    uint32_t key0, key1, stream_id;
    uint32_t sr, tiled, noclip;
};

// One tensor of a grouped launch: its tiles are workgroups [tile0, tile0 + row tiles x col_tiles).
struct DualItem {
    const void *x;
    int64_t ldx;
    uint32_t rows, cols, col_tiles, tile0;
    DualOut o1, o0;
};
struct DualGroup {
    DualItem item[kDualGroupMax];
    int count;
};

template <int H, bool F32, bool RHT, int NW>
__global__ __launch_bounds__(64 * NW) void quant_dual_kernel(DualGroup grp, float norm)
{
    static_assert(NW == 4 || NW == 8, "four or eight wavefronts");
    constexpr int kEsize = F32 ? 4 : 2;
    constexpr int kRowBytes = kDualTile * kEsize;
    constexpr int kParts = F32 ? 4 : 2;           // 16-byte pieces per 16-element group
    constexpr int kStepRows = 8 * NW;             // tile rows per row load of the workgroup
    constexpr int kSteps = kDualTile / kStepRows; // row loads per lane (8 rows per wavefront each)
    constexpr int kColsPerLane = 8 / NW;          // columns a lane quantizes in step 2
    __shared__ __attribute__((aligned(16))) uint8_t tile[kDualTile * kRowBytes];
    uint8_t *out = tile;                          // reused once the tile has been read
    uint8_t *out_scales = tile + kDualTile * 64;

    // the tensor of this workgroup: the last one whose first tile is at or below blockIdx.x (a
    // tensor without tiles shares its first tile with the next one)
    int it = 0;
    for (int i = 1; i < grp.count; ++i)
        if (blockIdx.x >= grp.item[i].tile0) it = i;
    const void *__restrict__ x = grp.item[it].x;
    const int64_t ldx = grp.item[it].ldx;
    const uint32_t rows = grp.item[it].rows, cols = grp.item[it].cols, col_tiles = grp.item[it].col_tiles;
    const DualOut o1 = grp.item[it].o1, o0 = grp.item[it].o0;
    const uint32_t t_index = blockIdx.x - grp.item[it].tile0;

    const uint32_t tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t c0 = (t_index % col_tiles) * kDualTile;
    const uint32_t r0 = (t_index / col_tiles) * kDualTile;
    const uint32_t nrows = min((uint32_t)kDualTile, rows - r0);  // multiples of 32
    const uint32_t ncols = min((uint32_t)kDualTile, cols - c0);
    const char *xb = reinterpret_cast<const char *>(x);

    // 1. load, keep, quantize along the rows
    {
        const uint32_t gi = lane % 8;           // 16-element group within the tile row
        const bool col_live = gi * 16 < ncols;  // a lane pair (one MX block) lives or dies whole
        const bool upper1 = lane & 1;
        // a lane outside the tensor loads an element inside it instead (row and group clamped):
        // the loads stay unconditional, and whatever it computes from them is never stored
        const uint32_t lg = min(gi, ncols / 16u - 1u);
        u32x4 raw[kSteps][kParts];
        if constexpr (!F32) {
            // coalesced: lane l loads half l / 32 of the group of lane l % 32 (rows 0-3 of the
            // step) and of lane 32 + l % 32 (rows 4-7); a swap pairs the halves (quant_rows)
            const uint32_t half = lane >> 5, ml = lane & 31u;
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const uint32_t lrA = min(kStepRows * k + 8u * wave + ml / 8u, nrows - 1u);
                const uint32_t lrB = min(kStepRows * k + 8u * wave + 4u + ml / 8u, nrows - 1u);
                const int64_t col = c0 + 16 * lg + 8 * half;
                const uint16_t *xh = reinterpret_cast<const uint16_t *>(xb);
                raw[k][0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xh + (int64_t)(r0 + lrA) * ldx + col));
                raw[k][1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(xh + (int64_t)(r0 + lrB) * ldx + col));
            }
#pragma unroll
            for (int k = 0; k < kSteps; ++k) pair_halves(raw[k][0], raw[k][1]);
        } else {
#pragma unroll
            for (int k = 0; k < kSteps; ++k) {
                const uint32_t lr = min(kStepRows * k + 8u * wave + lane / 8u, nrows - 1u);
                const u32x4 *src = reinterpret_cast<const u32x4 *>(xb + ((int64_t)(r0 + lr) * ldx + c0 + 16 * lg) * 4);
#pragma unroll
                for (int p = 0; p < kParts; ++p) raw[k][p] = __builtin_nontemporal_load(src + p);
            }
        }
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const uint32_t tr = kStepRows * k + 8 * wave + lane / 8;
            u32x4 *dst = reinterpret_cast<u32x4 *>(tile + tr * kRowBytes + gi * 16 * kEsize);
#pragma unroll
            for (int p = 0; p < kParts; ++p) dst[p] = raw[k][p];
        }
        // randomized rotation: this lane's 16 positions along the rows are the same for every k
        const uint32_t g1 = c0 / 16 + gi;
        const uint32_t row_signs =
            RHT ? (rht_sign_word(g1 / 2, o1.key0, o1.key1) >> (16 * (g1 % 2))) & 0xFFFFu : 0u;
#pragma unroll
        for (int k = 0; k < kSteps; ++k) {
            const uint32_t tr = kStepRows * k + 8 * wave + lane / 8;
            float v[16];
#pragma unroll
            for (int p = 0; p < kParts; ++p) {
                const uint32_t w[4] = {raw[k][p].x, raw[k][p].y, raw[k][p].z, raw[k][p].w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    if constexpr (F32) {
                        v[4 * p + u] = __uint_as_float(w[u]);
                    } else {
                        v[8 * p + 2 * u] = bf16_lo(w[u]);
                        v[8 * p + 2 * u + 1] = bf16_hi(w[u]);
                    }
                }
            }
            if constexpr (RHT) apply_signs<16>(v, row_signs);
            uint32_t amax;
            if constexpr (H == 16) {
                amax = fwht_regs_amax<16>(v);
                if (norm != 1.0f) {
                    scale_values<16>(v, norm);
                    amax = scaled_amax(amax, norm);
                }
            } else {
                if constexpr (H == 32) {
                    fwht_regs<16>(v);
                    fwht_cross_stage<1, 16>(v, upper1);
                    if (norm != 1.0f) scale_values<16>(v, norm);
                }
                amax = amax_bits<16>(v);
            }
            amax = max(amax, quad_xor<1>(amax));
            uint32_t sc = e8m0_from_amax_bits(amax);
            if (o1.noclip) sc = e8m0_noclip(amax, sc);
            const uint32_t o = r0 + tr, g = g1;   // quantized row, global 16-element group
            uint32_t w0, w1;
            prescale_if_zero_scale<16>(v, sc);
            const float div = e8m0_divisor(sc);
            if (o1.sr) {
                const uint64_t index0 = (uint64_t)o * cols + 16u * g;
                uint32_t w[2];
                encode_stochastic<2>(v, div, index0, o1.key0, o1.key1, o1.stream_id, w);
                w0 = w[0];
                w1 = w[1];
            } else {
                w0 = encode8_nearest(v, div);
                w1 = encode8_nearest(v + 8, div);
            }
            if (sc == 0xFFu) w0 = w1 = 0u;
            const u32x2 codes = {w0, w1};
            if (col_live && tr < nrows) {
                if (o1.tiled) {
                    const int64_t at = tiled_chunk(o, g / 2, cols) + 8 * (g % 2);
                    __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(o1.q + at));
                    if ((lane & 1u) == 0u) o1.scales[tiled_scale(o, g / 2, cols)] = (uint8_t)sc;
                } else {
                    __builtin_nontemporal_store(codes, reinterpret_cast<u32x2 *>(o1.q + (int64_t)o * o1.ldq) + g);
                    if ((lane & 1u) == 0u) o1.scales[(int64_t)o * o1.lds + g / 2] = (uint8_t)sc;
                }
            }
        }
    }
    __syncthreads();

    // 2. quantize along the columns: wavefront w takes the 32-row block w % 4; with four
    // wavefronts a lane takes two columns (bf16: the two halves of one LDS word), with eight one
    // column of the half w / 4 of the tile
    {
        const uint32_t blk = wave % 4, chalf = wave / 4;
        float v[kColsPerLane][32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint8_t *rowp = tile + (32 * blk + i) * kRowBytes;
            if constexpr (NW == 8) {
                const uint32_t tc = 64 * chalf + lane;
                if constexpr (F32)
                    v[0][i] = *reinterpret_cast<const float *>(rowp + 4 * tc);
                else
                    v[0][i] = __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(rowp + 2 * tc) << 16);
            } else if constexpr (F32) {
                v[0][i] = *reinterpret_cast<const float *>(rowp + 4 * lane);
                v[1][i] = *reinterpret_cast<const float *>(rowp + 4 * lane + 256);
            } else {
                const uint32_t w = *reinterpret_cast<const uint32_t *>(rowp + 4 * lane);
                v[0][i] = bf16_lo(w);
                v[1][i] = bf16_hi(w);
            }
        }
        __syncthreads();
        const uint32_t col_signs = RHT ? rht_sign_word(r0 / 32 + blk, o0.key0, o0.key1) : 0u;
#pragma unroll
        for (int cc = 0; cc < kColsPerLane; ++cc) {
            // tile column = quantized row
            const uint32_t tc = NW == 8 ? 64 * chalf + lane : (F32 ? lane + 64 * cc : 2 * lane + cc);
            if constexpr (RHT) apply_signs<32>(v[cc], col_signs);
            uint32_t amax = rotate_block_amax<H>(v[cc]);
            if (H > 0 && norm != 1.0f) {
                scale_values<32>(v[cc], norm);
                amax = scaled_amax(amax, norm);
            }
            uint32_t sc = e8m0_from_amax_bits(amax);
            if (o0.noclip) sc = e8m0_noclip(amax, sc);
            uint32_t words[4];
            prescale_if_zero_scale<32>(v[cc], sc);
            const float div = e8m0_divisor(sc);
            if (o0.sr) {
                const uint64_t index0 = (uint64_t)(c0 + tc) * rows + r0 + 32 * blk;
                encode_stochastic<4>(v[cc], div, index0, o0.key0, o0.key1, o0.stream_id, words);
            } else {
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) words[wd] = encode8_nearest(v[cc] + 8 * wd, div);
            }
            if (sc == 0xFFu) words[0] = words[1] = words[2] = words[3] = 0u;
            // tiled: 16-row slab, 64 bytes per row, chunk swizzled by (row % 16) / 4; the tile's
            // four blocks are chunks 0..3 of one 128-element slice (r0 is a multiple of 128)
            const uint32_t at = o0.tiled ? (tc / 16) * 1024 + (tc % 16) * 64 + 16 * (blk ^ ((tc % 16) / 4))
                                         : tc * 64 + 16 * blk;
            *reinterpret_cast<u32x4 *>(out + at) = u32x4{words[0], words[1], words[2], words[3]};
            out_scales[tc * 4 + blk] = (uint8_t)sc;
        }
    }
    __syncthreads();

    // 3. store the column output
    if (o0.tiled) {
        // rows % 512 == 0 here, so the tile has all four blocks; one 1 KB block per 16-row slab
#pragma unroll
        for (int pass = 0; pass < 8 / NW; ++pass) {
            const uint32_t s = NW * pass + wave;
            if (16 * s < ncols) {
                const u32x4 t = *reinterpret_cast<const u32x4 *>(out + s * 1024 + lane * 16);
                uint8_t *dst = o0.q + ((int64_t)(c0 / 16 + s) * (rows / 128) + r0 / 128) * 1024 + lane * 16;
                __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(dst));
            }
        }
        if (tid < ncols) {
            // the four scale bytes of quantized row o are adjacent (block r0/32 is a multiple of 4)
            const uint32_t o = c0 + tid;
            const uint32_t w = *reinterpret_cast<const uint32_t *>(out_scales + tid * 4);
            *reinterpret_cast<uint32_t *>(o0.scales + tiled_scale(o, r0 / 32, rows)) = w;
        }
    } else {
#pragma unroll
        for (int pass = 0; pass < 8 / NW; ++pass) {
            const uint32_t tc = 16 * NW * pass + tid / 4, blk = tid % 4;
            if (tc < ncols && 32 * blk < nrows) {
                const u32x4 t = *reinterpret_cast<const u32x4 *>(out + tc * 64 + 16 * blk);
                const int64_t o = c0 + tc;
                __builtin_nontemporal_store(t, reinterpret_cast<u32x4 *>(o0.q + o * o0.ldq + (r0 / 32 + blk) * 16));
                o0.scales[o * o0.lds + r0 / 32 + blk] = out_scales[tc * 4 + blk];
            }
        }
    }
}

template <int H, bool F32, bool RHT>
hipError_t dual_dispatch(const DualGroup &grp, uint32_t tiles, float norm, hipStream_t stream)
{
    return launch(quant_dual_kernel<H, F32, RHT, kDualWaves>, dim3(tiles), dim3(64 * kDualWaves), 0, stream, grp,
                  norm);
}

template <int H, bool F32, bool SR, bool TILED, bool RHT>
hipError_t rows_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         bool noclip, float norm, hipStream_t stream)
{
    const uint32_t gpr = (uint32_t)(cols / 16);
    const uint32_t total = (uint32_t)(rows * (cols / 16));
    const uint32_t per_block = kThreads * kRowsUnroll;
    const dim3 grid((total + per_block - 1) / per_block);
    return launch(quant_rows_kernel<H, F32, SR, TILED, RHT>, grid, dim3(kThreads), 0, stream, x, ldx, gpr, total, q,
                  ldq, scales, lds, (uint32_t)seed, (uint32_t)(seed >> 32), stream_id, cols, noclip ? 1u : 0u, norm,
                  (uint32_t)(rows - 1));
}

template <int H, bool F32, bool SR, bool TILED, bool RHT>
hipError_t cols_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         bool noclip, float norm, hipStream_t stream)
{
    const int64_t tile_cols = kColsRowBytes / (F32 ? 4 : 2);
    const int64_t col_tiles = (cols + tile_cols - 1) / tile_cols;
    const int64_t row_tiles = (rows + kColsTileRows - 1) / kColsTileRows;
    return launch(quant_cols_kernel<H, F32, SR, TILED, RHT>, dim3((unsigned)(col_tiles * row_tiles)), dim3(kThreads), 0,
                  stream, x, ldx, (uint32_t)rows, (uint32_t)cols, (uint32_t)col_tiles, q, ldq, scales, lds,
                  (uint32_t)seed, (uint32_t)(seed >> 32), stream_id, noclip ? 1u : 0u, norm);
}

// orthonormal rotation (hadamard | kOrthonormal): the binary32 number nearest to 1/sqrt(h) that
// multiplies every rotated value (h = 16: 1/4 exactly; h = 32: 2^-2.5 = sqrt(2) / 8 rounded to
// binary32); 1 for the unnormalised H, which the kernels skip
float rotation_norm(int hadamard)
{
    if (!(hadamard & kOrthonormal)) return 1.0f;
    return (hadamard & kHadamardSize) == 16 ? 0.25f : 0x1.6a09e6p-3f;
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

// the randomized variants exist only for H = 16 and 32 (the entry points reject RHT with H = 0)
template <int H, bool F32, bool SR>
struct RowsSel {
    template <typename... A>
    static hipError_t run(bool tiled, bool rht, A... a)
    {
        if constexpr (H > 0) {
            if (rht) return tiled ? rows_dispatch<H, F32, SR, true, true>(a...) : rows_dispatch<H, F32, SR, false, true>(a...);
        }
        return tiled ? rows_dispatch<H, F32, SR, true, false>(a...) : rows_dispatch<H, F32, SR, false, false>(a...);
    }
};

template <int H, bool F32, bool SR>
struct ColsSel {
    template <typename... A>
    static hipError_t run(bool tiled, bool rht, A... a)
    {
        if constexpr (H > 0) {
            if (rht) return tiled ? cols_dispatch<H, F32, SR, true, true>(a...) : cols_dispatch<H, F32, SR, false, true>(a...);
        }
        return tiled ? cols_dispatch<H, F32, SR, true, false>(a...) : cols_dispatch<H, F32, SR, false, false>(a...);
    }
};

}  // namespace

hipError_t launch_quantize_rows(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, bool noclip, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<RowsSel>(hadamard & kHadamardSize, f32, stochastic, tiled, (hadamard & kRandomizedHadamard) != 0,
                         x, rows, cols, ldx, seed, stream_id, q, ldq, scales, lds, noclip, rotation_norm(hadamard),
                         stream);
}

hipError_t launch_quantize_cols(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, bool noclip, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<ColsSel>(hadamard & kHadamardSize, f32, stochastic, tiled, (hadamard & kRandomizedHadamard) != 0,
                         x, rows, cols, ldx, seed, stream_id, q, ldq, scales, lds, noclip, rotation_norm(hadamard),
                         stream);
}

hipError_t launch_quantize_dual_grouped(const DualInput *items, int count, bool f32, int hadamard,
                                        hipStream_t stream)
{
    if (count < 1 || count > kDualGroupMax) return hipErrorInvalidValue;
    const auto conv = [](const QuantOut &o) {
        return DualOut{o.q, o.ldq, o.scales, o.lds, (uint32_t)o.seed, (uint32_t)(o.seed >> 32), o.stream_id,
                       o.stochastic ? 1u : 0u, o.tiled ? 1u : 0u, o.noclip ? 1u : 0u};
    };
    DualGroup grp{};
    grp.count = count;
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        const DualInput &d = items[i];
        const int64_t col_tiles = (d.cols + kDualTile - 1) / kDualTile;
        const int64_t row_tiles = (d.rows + kDualTile - 1) / kDualTile;
        grp.item[i] = DualItem{d.x, d.ldx, (uint32_t)d.rows, (uint32_t)d.cols, (uint32_t)col_tiles, (uint32_t)tiles,
                               conv(d.axis1), conv(d.axis0)};
        tiles += d.rows > 0 && d.cols > 0 ? col_tiles * row_tiles : 0;
    }
    if (tiles == 0) return hipSuccess;
    if (tiles > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    const float norm = rotation_norm(hadamard);
    const bool rht = (hadamard & kRandomizedHadamard) != 0;
    const uint32_t n = (uint32_t)tiles;
    switch ((hadamard & kHadamardSize) * 4 + (f32 ? 2 : 0) + (rht ? 1 : 0)) {
    case 0: return dual_dispatch<0, false, false>(grp, n, norm, stream);
    case 2: return dual_dispatch<0, true, false>(grp, n, norm, stream);
    case 64: return dual_dispatch<16, false, false>(grp, n, norm, stream);
    case 65: return dual_dispatch<16, false, true>(grp, n, norm, stream);
    case 66: return dual_dispatch<16, true, false>(grp, n, norm, stream);
    case 67: return dual_dispatch<16, true, true>(grp, n, norm, stream);
    case 128: return dual_dispatch<32, false, false>(grp, n, norm, stream);
    case 129: return dual_dispatch<32, false, true>(grp, n, norm, stream);
    case 130: return dual_dispatch<32, true, false>(grp, n, norm, stream);
    case 131: return dual_dispatch<32, true, true>(grp, n, norm, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_quantize_dual(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, const QuantOut &axis1, const QuantOut &axis0,
                                hipStream_t stream)
{
    const DualInput one{x, rows, cols, ldx, axis1, axis0};
    return launch_quantize_dual_grouped(&one, 1, f32, hadamard, stream);
}

}  // namespace mx

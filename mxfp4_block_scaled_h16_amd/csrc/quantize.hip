// Fused rotate + amax + E8M0 scale + E2M1 encode + pack kernels (gfx950).
//
// The operand transform of the gist.science summary of "MXFP4 LLM pretraining", section 방법론
// (Methodology): deterministic block Hadamard (H16 / H32) along the GEMM's contraction axis, then
// MXFP4 quantization with nearest-even or stochastic rounding. Two kernels:
//   quant_rows -- along the contiguous axis (Fprop operands, the Dgrad gradient operand);
//   quant_cols -- along the strided axis, writing the quantized transpose (the Wgrad token axis,
//                 section "주요 기여 및 발견" §1: the weight gradient is where MXFP4 hurts most).
// Both are HBM-bound: 2 bytes read and 0.5 + 1/32 bytes written per bf16 element.
#include "internal.h"
#include "mx_device.h"

namespace mx {
namespace {

constexpr int kThreads = 256;

// Load the 32 elements of the MX block at p (contiguous) into v as binary32.
template <bool F32>
__device__ __forceinline__ void load_block_contiguous(const void *p, float *v)
{
    if constexpr (F32) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(p);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const f32x4 t = __builtin_nontemporal_load(src + j);
            v[4 * j + 0] = t.x;
            v[4 * j + 1] = t.y;
            v[4 * j + 2] = t.z;
            v[4 * j + 3] = t.w;
        }
    } else {
        const u32x4 *src = reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const u32x4 t = __builtin_nontemporal_load(src + j);
            const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                v[8 * j + 2 * u] = bf16_lo(w[u]);
                v[8 * j + 2 * u + 1] = bf16_hi(w[u]);
            }
        }
    }
}

// One thread per MX block along a row: rows x (cols / 32) blocks in total.
template <int H, bool F32, bool SR>
__global__ __launch_bounds__(kThreads) void quant_rows_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t blocks_per_row, uint32_t total_blocks,
    uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales, int64_t lds, uint32_t key0,
    uint32_t key1, uint32_t stream_id, int64_t L)
{
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= total_blocks) return;
    const uint32_t r = g / blocks_per_row;
    const uint32_t b = g - r * blocks_per_row;
    const size_t esize = F32 ? 4 : 2;
    const char *src = reinterpret_cast<const char *>(x) + ((int64_t)r * ldx + (int64_t)b * 32) * esize;
    float v[32];
    load_block_contiguous<F32>(src, v);
    rotate_block<H>(v);
    uint32_t words[4];
    const uint64_t index0 = (uint64_t)r * (uint64_t)L + (uint64_t)b * 32u;
    const uint32_t s = encode_block<SR>(v, words, index0, key0, key1, stream_id);
    uint4 out;
    out.x = words[0];
    out.y = words[1];
    out.z = words[2];
    out.w = words[3];
    *reinterpret_cast<uint4 *>(q + (int64_t)r * ldq + (int64_t)b * 16) = out;
    scales[(int64_t)r * lds + b] = (uint8_t)s;
}

// One thread per (column pair, run of RB consecutive 32-row blocks). Each loaded row gives the
// thread two adjacent columns (4 bytes of bf16 / 8 bytes of f32); adjacent threads take adjacent
// column pairs, so each row read by a wavefront is one contiguous segment.
template <int H, bool F32, bool SR, int RB>
__global__ __launch_bounds__(kThreads) void quant_cols_kernel(
    const void *__restrict__ x, int64_t ldx, uint32_t cols, uint32_t col_pairs, uint32_t row_runs,
    uint32_t row_blocks, uint8_t *__restrict__ q, int64_t ldq, uint8_t *__restrict__ scales,
    int64_t lds, uint32_t key0, uint32_t key1, uint32_t stream_id, int64_t L)
{
    const uint32_t g = blockIdx.x * kThreads + threadIdx.x;
    if (g >= col_pairs * row_runs) return;
    const uint32_t run = g / col_pairs;
    const uint32_t cp = g - run * col_pairs;
    const uint32_t c0 = 2 * cp;
    const bool has_second = c0 + 1 < cols;
#pragma unroll 1
    for (int rbi = 0; rbi < RB; ++rbi) {
        const uint32_t rb = run * RB + rbi;
        if (rb >= row_blocks) break;
        float v0[32], v1[32];
        if constexpr (F32) {
            const float *base = reinterpret_cast<const float *>(x) + (int64_t)rb * 32 * ldx + c0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                if (has_second) {
                    const f32x2 t = __builtin_nontemporal_load(reinterpret_cast<const f32x2 *>(base + (int64_t)i * ldx));
                    v0[i] = t.x;
                    v1[i] = t.y;
                } else {
                    v0[i] = __builtin_nontemporal_load(base + (int64_t)i * ldx);
                    v1[i] = 0.0f;
                }
            }
        } else {
            const uint16_t *base = reinterpret_cast<const uint16_t *>(x) + (int64_t)rb * 32 * ldx + c0;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                uint32_t w;
                if (has_second) {
                    w = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(base + (int64_t)i * ldx));
                } else {
                    w = __builtin_nontemporal_load(base + (int64_t)i * ldx);
                }
                v0[i] = bf16_lo(w);
                v1[i] = bf16_hi(w);
            }
        }
        rotate_block<H>(v0);
        rotate_block<H>(v1);
        uint32_t w0[4], w1[4];
        const uint64_t idx0 = (uint64_t)c0 * (uint64_t)L + (uint64_t)rb * 32u;
        const uint32_t s0 = encode_block<SR>(v0, w0, idx0, key0, key1, stream_id);
        *reinterpret_cast<uint4 *>(q + (int64_t)c0 * ldq + (int64_t)rb * 16) = make_uint4(w0[0], w0[1], w0[2], w0[3]);
        scales[(int64_t)c0 * lds + rb] = (uint8_t)s0;
        if (has_second) {
            const uint32_t s1 = encode_block<SR>(v1, w1, idx0 + (uint64_t)L, key0, key1, stream_id);
            *reinterpret_cast<uint4 *>(q + (int64_t)(c0 + 1) * ldq + (int64_t)rb * 16) = make_uint4(w1[0], w1[1], w1[2], w1[3]);
            scales[(int64_t)(c0 + 1) * lds + rb] = (uint8_t)s1;
        }
    }
}

template <int H, bool F32, bool SR>
hipError_t rows_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         hipStream_t stream)
{
    const uint32_t bpr = (uint32_t)(cols / 32);
    const uint32_t total = (uint32_t)(rows * (cols / 32));
    const dim3 grid((total + kThreads - 1) / kThreads);
    return launch(quant_rows_kernel<H, F32, SR>, grid, dim3(kThreads), 0, stream, x, ldx, bpr, total,
                  q, ldq, scales, lds, (uint32_t)seed, (uint32_t)(seed >> 32), stream_id, cols);
}

template <int H, bool F32, bool SR>
hipError_t cols_dispatch(const void *x, int64_t rows, int64_t cols, int64_t ldx, uint64_t seed,
                         uint32_t stream_id, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                         hipStream_t stream)
{
    constexpr int RB = 4;
    const uint32_t row_blocks = (uint32_t)(rows / 32);
    const uint32_t row_runs = (row_blocks + RB - 1) / RB;
    const uint32_t col_pairs = (uint32_t)((cols + 1) / 2);
    const uint32_t total = col_pairs * row_runs;
    const dim3 grid((total + kThreads - 1) / kThreads);
    return launch(quant_cols_kernel<H, F32, SR, RB>, grid, dim3(kThreads), 0, stream, x, ldx,
                  (uint32_t)cols, col_pairs, row_runs, row_blocks, q, ldq, scales, lds,
                  (uint32_t)seed, (uint32_t)(seed >> 32), stream_id, rows);
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
    static hipError_t run(A... a) { return rows_dispatch<H, F32, SR>(a...); }
};

template <int H, bool F32, bool SR>
struct ColsSel {
    template <typename... A>
    static hipError_t run(A... a) { return cols_dispatch<H, F32, SR>(a...); }
};

}  // namespace

hipError_t launch_quantize_rows(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, uint64_t seed, uint32_t stream_id,
                                uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<RowsSel>(hadamard, f32, stochastic, x, rows, cols, ldx, seed, stream_id, q, ldq,
                         scales, lds, stream);
}

hipError_t launch_quantize_cols(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, uint64_t seed, uint32_t stream_id,
                                uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream)
{
    return pick<ColsSel>(hadamard, f32, stochastic, x, rows, cols, ldx, seed, stream_id, q, ldq,
                         scales, lds, stream);
}

}  // namespace mx

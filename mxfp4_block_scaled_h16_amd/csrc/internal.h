// Launchers shared by the C-ABI entry points (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

// hadamard argument of the launchers: the size (0, 16, 32) in the low byte, plus the
// randomized-Hadamard flag (the public MXFP4_RHT) and the orthonormal flag.
constexpr int kHadamardSize = 0xFF;
constexpr int kRandomizedHadamard = 0x100;
constexpr int kOrthonormal = 0x200;  // rotate by H_h / sqrt(h) (the public MXFP4_ORTHONORMAL)

// Arguments are validated by the caller; these only pick a kernel and enqueue it.
// tiled: write the tiled layout (L % 512 == 0; ldq and lds unused), else row-major.
hipError_t launch_quantize_rows(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, bool noclip, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream);

hipError_t launch_quantize_cols(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, bool stochastic, bool noclip, uint64_t seed, uint32_t stream_id,
                                bool tiled, uint8_t *q, int64_t ldq, uint8_t *scales, int64_t lds,
                                hipStream_t stream);

// One output of launch_quantize_dual: the same arguments launch_quantize_rows/cols take.
struct QuantOut {
    bool stochastic;
    bool noclip;
    uint64_t seed;
    uint32_t stream_id;
    bool tiled;
    uint8_t *q;
    int64_t ldq;
    uint8_t *scales;
    int64_t lds;
};

// Both quantizations of x[rows][cols] from one read: axis1 = launch_quantize_rows' output,
// axis0 = launch_quantize_cols' output, bit-identical to the two separate launches.
// Requires rows % 32 == 0 and cols % 32 == 0 (and the tiled outputs' lengths % 512 == 0).
hipError_t launch_quantize_dual(const void *x, bool f32, int64_t rows, int64_t cols, int64_t ldx,
                                int hadamard, const QuantOut &axis1, const QuantOut &axis0,
                                hipStream_t stream);

// Several tensors' dual quantizations in one launch (one element type and rotation, up to 8
// tensors of any shapes): every tensor's 128 x 128 tiles are workgroups of the same grid.
constexpr int kDualGroupMax = 8;
struct DualInput {
    const void *x;
    int64_t rows, cols, ldx;
    QuantOut axis1, axis0;
};
hipError_t launch_quantize_dual_grouped(const DualInput *items, int count, bool f32, int hadamard,
                                        hipStream_t stream);

// tiled: both operands in the tiled layout (K % 512 == 0, rows padded to multiples of 256);
// otherwise row-major with leading dimensions. A workspace of gemm_workspace_bytes() bytes
// (16-byte aligned) lets a GEMM with few output tiles split K (gemm_splits() ways) into FP32
// partials that a second kernel sums in fixed order; without it the GEMM runs unsplit.
// c = alpha * A B^T + beta * c, FP32 (bf16 = false) or bf16 (round to nearest even); c is not
// read when beta == 0. beta == 0 with FP32 output runs the FP32-only kernel instantiation.
hipError_t launch_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                       const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs, int64_t M,
                       int64_t N, int64_t K, float alpha, float beta, void *c, bool bf16, int64_t ldc,
                       bool tiled, void *workspace, size_t ws_bytes, hipStream_t stream);
int gemm_splits(int64_t M, int64_t N, int64_t K);

// Several products of the same shape, strides and layout in one launch (FP32 output, alpha,
// beta 0, no split of K): one grid over all their tiles, so that products with few tiles fill
// the chip together. Where the pipelined kernel does not apply (K % 512 != 0 row-major
// operands) the row kernel runs them as the layers of a three-dimensional grid; more than 8
// products fall back to one launch each.
struct GemmGroupItem {
    const uint8_t *aq, *as, *bq, *bs;
    float *c;
};
hipError_t launch_gemm_grouped(const GemmGroupItem *items, int count, int64_t lda, int64_t ldas, int64_t ldb,
                               int64_t ldbs, int64_t M, int64_t N, int64_t K, float alpha, int64_t ldc, bool tiled,
                               hipStream_t stream);
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

// c[m][n] = 0 for m < M, n < N (a kernel, not a memset, so it is safe inside captured graphs).
// K == 0: c = beta * c (zeros when beta == 0, c not read)
hipError_t launch_empty_product(void *c, bool bf16, int64_t M, int64_t N, int64_t ldc, float beta,
                                hipStream_t stream);

// Launch a kernel through hipLaunchKernel so the runtime's error comes back directly.
template <typename... Params, typename... Args>
hipError_t launch(void (*kernel)(Params...), dim3 grid, dim3 block, size_t shared, hipStream_t stream,
                  Args... args)
{
    static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
    auto pack = [&](auto... typed) {
        void *argv[] = {(void *)&typed...};
        return hipLaunchKernel((const void *)kernel, grid, block, argv, shared, stream);
    };
    return pack(static_cast<Params>(args)...);
}

}  // namespace mx

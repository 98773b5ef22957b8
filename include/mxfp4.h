/*
 * mxfp4.h -- C ABI of the MXFP4 + block-Hadamard linear-layer library for AMD MI355X (gfx950).
 *
 * What it computes. The gist.science summary of "MXFP4 LLM pretraining" (Llama-3.1-8B on
 * MI355X), section 방법론 (Methodology), runs all three GEMMs of a linear layer in MXFP4 -- the
 * forward product (Fprop), the activation gradient (Dgrad) and the weight gradient (Wgrad) -- and
 * stabilises them with a deterministic 16x16 or 32x32 Hadamard rotation of the operands before
 * quantization (section "주요 기여 및 발견" §2: the deterministic H16 on the whole pipeline is
 * what restores convergence; stochastic rounding is the other intervention it tries).
 *
 * MXFP4 here (OCP Microscaling Formats v1.0): blocks of 32 consecutive elements along the
 * quantized axis share one E8M0 scale byte S (value 2^(S-127); 0xFF = NaN) and each element is an
 * E2M1 code (sign bit 3, magnitude index into {0, .5, 1, 1.5, 2, 3, 4, 6}). Two codes per byte,
 * the even element in the low nibble (molayo1419.me NVFP4 article, "주요 사실": two 4-bit values
 * packed into one byte).
 *
 * Conventions fixed by this library (the pages leave them open):
 *  - H_h is the unnormalised Sylvester Hadamard H[i][j] = (-1)^popcount(i&j), applied to each
 *    aligned group of h consecutive elements along the quantized axis, as a binary32 fast
 *    Walsh-Hadamard transform with strides 1, 2, 4, ... and pair update (u, w) -> (u+w, u-w).
 *    Since H_h H_h^T = h I, GEMMs of rotated operands are scaled by alpha = 1/h.
 *  - Scale byte: S = floor(log2(amax)) - 2 + 127 clamped to [0, 254]; 0xFF (and all codes 0)
 *    when the block holds a NaN or infinity after rotation; 0 for an all-zero block.
 *  - Nearest rounding: ties to the even code, saturation at 6; the sign bit follows the sign
 *    of the rotated value, also for zero results.
 *  - Stochastic rounding: |v| >= 6 saturates; otherwise rounds up to the next grid value iff
 *    floor(r / 2^10) < floor(2^22 (|v| - lo) / (hi - lo)) (22 random bits against the
 *    fractional position truncated to 22 bits, the rule of gfx950's stochastic FP4
 *    conversion), r = word (i mod 4) of Philox4x32-10 (Salmon et al., SC'11)
 *    with key (seed mod 2^32, seed >> 32) and counter (floor(i/4) mod 2^32, floor(i/4) >> 32,
 *    stream, 0), where i = o * L + j is the element's position in the quantized output
 *    (row o of the output, position j along the quantized axis of length L).
 *
 * Memory and execution conventions (every entry point):
 *  - All tensor pointers are DEVICE pointers, row-major, owned by the caller. The library never
 *    allocates, frees or retains them. `stream` is a hipStream_t passed as void* (NULL = the
 *    default stream); work is enqueued asynchronously and the call returns before it finishes.
 *  - Argument errors are detected before any launch: the call returns the error code, launches
 *    nothing and leaves every output untouched. A failed launch returns MXFP4_ERR_LAUNCH.
 *    Nothing aborts and nothing throws across this interface.
 *  - No hidden state: calls are reentrant. Results are deterministic run to run (quantization
 *    bit-exact; GEMMs accumulate in a fixed order, no atomics).
 *  - The device current on the calling thread must be a gfx950 GPU (else MXFP4_ERR_DEVICE).
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Raised whenever an entry point, a struct or the bits an entry point produces change. 12:
 * mxfp4_quantize_dual_grouped and mxfp4_dual_item_t. 11: mxfp4_gemm_grouped and
 * mxfp4_gemm_item_t. 10:
 * mxfp4_linear_fprop_noalloc; GEMMs whose contraction exceeds 5120 accumulate in fixed segments
 * (their FP32 results differ from 9 in the last bits); every enum spans the int32 range. 9: the
 * stochastic-rounding decision compares 22 random bits with the fractional position truncated to
 * 22 bits (codes for |v| < 1 differ from 8). */
#define MXFP4_ABI_VERSION 12

/* Every enum below includes the whole int32 range (the _RANGE_ members are not values to pass):
 * an entry point receives whatever integer a C caller passes and refuses the ones it does not
 * define with MXFP4_ERR_ARG, which in C++ is only well defined when the enum type can hold it. */
#define MXFP4_ENUM_RANGE(prefix) prefix##_RANGE_MIN_ = -0x7FFFFFFF - 1, prefix##_RANGE_MAX_ = 0x7FFFFFFF

typedef enum {
    MXFP4_OK = 0,
    MXFP4_ERR_NULL = 1,      /* a required pointer is NULL */
    MXFP4_ERR_SHAPE = 2,     /* a size is negative, or a quantized / contraction length % 32 != 0 */
    MXFP4_ERR_ARG = 3,       /* bad enum, hadamard not in {0,16,32}, ld smaller than the row */
    MXFP4_ERR_ALIGN = 4,     /* pointer or leading dimension misaligned (see each call) */
    MXFP4_ERR_WORKSPACE = 5, /* workspace smaller than mxfp4_linear_workspace_bytes() */
    MXFP4_ERR_DEVICE = 6,    /* no current HIP device, or it is not gfx950 */
    MXFP4_ERR_LAUNCH = 7,    /* the HIP runtime reported a launch error */
    MXFP4_ENUM_RANGE(MXFP4_STATUS)
} mxfp4_status_t;

typedef enum { MXFP4_IN_BF16 = 0, MXFP4_IN_F32 = 1, MXFP4_ENUM_RANGE(MXFP4_DTYPE) } mxfp4_dtype_t;

typedef enum { MXFP4_RNE = 0, MXFP4_SR_PHILOX = 1, MXFP4_ENUM_RANGE(MXFP4_ROUNDING) } mxfp4_rounding_t;

/*
 * Scale variant: OR into a rounding value (quantize, quantize_dual, linear cfg rnd_a / rnd_b) to
 * use the smallest scale that maps the block maximum to at most 6 -- S + 1 exactly when
 * amax > 6 * 2^(S - 127) -- so no element of the block saturates, instead of the OCP rule
 * S = floor(log2 amax) - 2 whose block maximum can map into [6, 8) and clip to 6. The pages fix
 * neither; the default follows the OCP MX specification.
 */
#define MXFP4_SCALE_NOCLIP 0x10

typedef enum { MXFP4_FPROP = 0, MXFP4_DGRAD = 1, MXFP4_WGRAD = 2, MXFP4_ENUM_RANGE(MXFP4_PASS) } mxfp4_pass_t;

/*
 * Randomized Hadamard: OR this flag into a hadamard size of 16 or 32 (quantize, quantize_dual,
 * linear cfg) to rotate y = H_h (d .* x) instead of y = H_h x. d_j = -1 or +1 for position j
 * along the quantized axis, the same for every quantized row: d_j = -1 iff bit (j mod 32) of word
 * ((j / 32) mod 4) of Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter
 * (floor(j/128) mod 2^32, floor(j/128) >> 32, 0, 1). The two operands of one GEMM must use the
 * same seed; the product then keeps the factor h (alpha = 1/h). Defined by: the Methodology
 * section names randomized Hadamard rotations as the other rotation tried (and reports that it
 * did not converge on the full pipeline); the construction is this library's reading.
 */
#define MXFP4_RHT 0x100

/*
 * Orthonormal rotation: OR this flag into a hadamard size of 16 or 32 (with or without
 * MXFP4_RHT) to rotate by H_h / sqrt(h) instead of H_h. The binary32 transform is followed by one
 * binary32 multiplication of every rotated value by the binary32 number nearest to 1/sqrt(h)
 * (1/4 for h = 16, exact: the codes are those of H16 and every scale byte is 2 lower; 2^-2.5
 * rounded for h = 32, which changes the rounding). A product of two such operands needs no 1/h
 * factor, so the linear entry points use alpha = 1. The pages (gist.science summary of "MXFP4
 * LLM pretraining", section 방법론) name 16x16 and 32x32 Hadamard matrices without a
 * normalisation; the unnormalised H with alpha = 1/h is this library's default reading.
 */
#define MXFP4_ORTHONORMAL 0x200

/*
 * Memory layout of a quantized operand with `outer` quantized rows of length L.
 *
 * MXFP4_LAYOUT_ROWS: row-major. codes q[outer][ldq] bytes (the first L/2 used: element j of row o
 *   is nibble j % 2 of byte j / 2, even element in the low nibble), scales s[outer][lds] bytes
 *   (the first L/32 used: block c covers elements [32 c, 32 c + 32)).
 * MXFP4_LAYOUT_TILED: the layout the GEMM streams without reshuffling; requires L % 512 == 0.
 *   Rows are padded to R = 256 * ceil(outer / 256); the padding is never written and only feeds
 *   outputs that are discarded. With the same nibble packing inside each 16-byte chunk:
 *     codes (R * L / 2 bytes): the chunk holding block c of row o starts at byte
 *       ((o / 16) * (L / 128) + c / 4) * 1024 + (o % 16) * 64 + 16 * ((c % 4) ^ ((o % 16) / 4));
 *     scales (R * L / 32 bytes): the scale of block c of row o is byte
 *       ((o / 64) * (L / 512) + c / 16) * 1024 + (o % 64) * 16 + (c % 16).
 *   Every 16-row x 128-element slice of codes and every 64-row x 512-element slice of scales is
 *   one contiguous kilobyte. Both pointers must be 16-byte aligned; ldq and lds are not used.
 */
typedef enum { MXFP4_LAYOUT_ROWS = 0, MXFP4_LAYOUT_TILED = 1, MXFP4_ENUM_RANGE(MXFP4_LAYOUT) } mxfp4_layout_t;

/* Bytes of codes and of scales of a tiled operand (outer rows, length L); MXFP4_ERR_SHAPE if
 * L % 512 != 0 or a size is negative, MXFP4_ERR_NULL if an output pointer is NULL. */
mxfp4_status_t mxfp4_tiled_sizes(int64_t outer, int64_t L, size_t *codes_bytes, size_t *scales_bytes);

/*
 * mxfp4_quantize -- rotate then quantize a 2-D tensor to MXFP4.
 *
 * Defined by: the operand transform of the Methodology section (deterministic H16/H32 rotation,
 * then MXFP4 with nearest or stochastic rounding), with the conventions above.
 *
 *   x        device, T[rows][cols] with row stride ldx elements; dtype bf16 or f32.
 *   axis=1   quantize along each row (L = cols):   q[rows][ldq bytes, first cols/2 used],
 *                                                  scales[rows][lds bytes, first cols/32 used].
 *   axis=0   quantize along each column (L = rows) and write the quantized TRANSPOSE:
 *                                                  q[cols][ldq], scales[cols][lds]
 *            (the Wgrad token axis and the Dgrad weight operand).
 *   hadamard 0 (no rotation), 16 or 32, or 16 / 32 | MXFP4_RHT (randomized, signs keyed by seed)
 *            and / or | MXFP4_ORTHONORMAL (H_h / sqrt(h));
 *            rounding MXFP4_RNE or MXFP4_SR_PHILOX with (seed, stream).
 *   layout   MXFP4_LAYOUT_ROWS (q, ldq, scales, lds as above) or MXFP4_LAYOUT_TILED (see above).
 *
 * Requirements: rows, cols >= 0; L % 32 == 0; at most 2^30 32-element blocks (rows * cols / 32);
 * rows layout: ldx >= cols; ldq >= L/2; lds >= L/32. Tiled layout: L % 512 == 0.
 * Alignment: x 16-byte aligned and ldx * sizeof(element) a multiple of 16; q 16-byte aligned and
 * (rows layout) ldq % 16 == 0; (tiled layout) scales 16-byte aligned. Empty tensors return
 * MXFP4_OK without a launch.
 */
mxfp4_status_t mxfp4_quantize(const void *x, mxfp4_dtype_t dtype, int64_t rows, int64_t cols,
                              int64_t ldx, int axis, int hadamard, mxfp4_rounding_t rounding,
                              uint64_t seed, uint32_t stream_id, mxfp4_layout_t layout, uint8_t *q,
                              int64_t ldq, uint8_t *scales, int64_t lds, void *stream);

/* One output of mxfp4_quantize_dual: what mxfp4_quantize takes for that axis. */
typedef struct {
    mxfp4_rounding_t rounding;
    uint64_t seed;
    uint32_t stream_id;
    mxfp4_layout_t layout;
    uint8_t *q;
    int64_t ldq;
    uint8_t *scales;
    int64_t lds;
} mxfp4_quant_out_t;

/*
 * mxfp4_quantize_dual -- both quantizations of one tensor from a single read of it.
 *
 * Defined by: the operand transform of the Methodology section, as for mxfp4_quantize. That
 * section runs all three GEMMs in MXFP4, so each of X, W and dY is a contraction operand along
 * both of its axes (X: Fprop along K, Wgrad along the tokens; W: Fprop along K, Dgrad along N;
 * dY: Dgrad along N, Wgrad along the tokens). This call writes both from one pass over x and is
 * bit-identical to the two calls
 *   mxfp4_quantize(x, dtype, rows, cols, ldx, 1, hadamard, <out_axis1 fields>, stream) and
 *   mxfp4_quantize(x, dtype, rows, cols, ldx, 0, hadamard, <out_axis0 fields>, stream).
 * Requirements: those of both calls (so rows % 32 == 0 and cols % 32 == 0); the two outputs must
 * not overlap each other or x. Per bf16 element it reads 2 bytes instead of 4.
 */
mxfp4_status_t mxfp4_quantize_dual(const void *x, mxfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                   int64_t ldx, int hadamard, const mxfp4_quant_out_t *out_axis1,
                                   const mxfp4_quant_out_t *out_axis0, void *stream);

/* One tensor of mxfp4_quantize_dual_grouped: the arguments mxfp4_quantize_dual takes for it. */
typedef struct {
    const void *x;
    mxfp4_dtype_t dtype;
    int64_t rows, cols, ldx;
    mxfp4_quant_out_t axis1, axis0;
} mxfp4_dual_item_t;

#define MXFP4_DUAL_GROUP_MAX 8

/*
 * mxfp4_quantize_dual_grouped -- the dual quantizations of up to MXFP4_DUAL_GROUP_MAX tensors
 * in one launch.
 *
 * Defined by: mxfp4_quantize_dual (Methodology section), for each item; the outputs are bitwise
 * those of the separate calls. It serves the operands a training step quantizes back to back
 * (an activation and the weight of the product that reads it, the key and value weights), so
 * that small tensors share one grid instead of each leaving most of the chip idle.
 *   items    host array of count entries, read before the call returns; each as
 *            mxfp4_quantize_dual requires it; every item has the same dtype; no output may
 *            overlap another output or any input.
 *   count    0 .. MXFP4_DUAL_GROUP_MAX (0: nothing to do).
 * Errors: MXFP4_ERR_ARG for count out of range or mixed dtypes; otherwise those of
 * mxfp4_quantize_dual, for the first item that fails them (nothing is launched then).
 */
mxfp4_status_t mxfp4_quantize_dual_grouped(const mxfp4_dual_item_t *items, int count, int hadamard,
                                           void *stream);

/*
 * mxfp4_gemm -- block-scaled FP4 GEMM with FP32 accumulation and output.
 *
 * Defined by: the MXFP4 GEMMs of the Methodology section, run natively on the FP4 matrix cores.
 *   c[m][n] = alpha * sum_k deq(A)[m][k] * deq(B)[n][k],  m < M, n < N, k < K,
 * with A = (aq [M][lda bytes], as [M][ldas bytes]) and B = (bq [N][ldb], bs [N][ldbs]) both
 * quantized along K (the layout mxfp4_quantize writes), deq(code, S) = e2m1(code) * 2^(S-127).
 * Any 0xFF scale in the contributing blocks makes the output NaN.
 * c is FP32 [M][ldc] (device). Requirements: M, N, K >= 0, K % 32 == 0, ldc >= N. Rows layout:
 * lda, ldb >= K/2 and multiples of 16, ldas, ldbs >= K/32, aq, bq 16-byte aligned. Tiled layout
 * (both operands, as mxfp4_quantize writes it with L = K): K % 512 == 0, all four operand
 * pointers 16-byte aligned, the leading dimensions unused.
 * workspace (optional, device, 16-byte aligned, ws_bytes >= mxfp4_gemm_workspace_bytes()): lets a
 * product with few output tiles split its contraction into FP32 partials that a second kernel
 * adds in a fixed order (deterministic); with workspace == NULL or too small it runs unsplit.
 * The workspace is in use until the enqueued work finishes.
 */
mxfp4_status_t mxfp4_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                          const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs,
                          int64_t M, int64_t N, int64_t K, float alpha, float *c, int64_t ldc,
                          mxfp4_layout_t layout, void *workspace, size_t ws_bytes, void *stream);

/* Output element type of mxfp4_gemm_ex. */
typedef enum { MXFP4_OUT_F32 = 0, MXFP4_OUT_BF16 = 1, MXFP4_ENUM_RANGE(MXFP4_OUT) } mxfp4_out_dtype_t;

/*
 * mxfp4_gemm_ex -- mxfp4_gemm with an epilogue: c = alpha * A B^T + beta * c.
 *
 * Defined by: the same product as mxfp4_gemm (Methodology section). The extra terms serve the
 * training step around it: beta = 1 accumulates a weight gradient into an existing FP32 buffer
 * (gradient accumulation over micro-batches), and a bf16 output halves the bytes of an
 * activation-sized result.
 *   c        device, c_dtype[M][ldc]: MXFP4_OUT_F32 (4-byte aligned) or MXFP4_OUT_BF16 (2-byte
 *            aligned; the FP32 result is rounded to nearest even once, after beta * c is added).
 *   beta     c is read only when beta != 0 (it may then hold anything, even NaN, when beta == 0).
 * The sum alpha * acc + beta * c is formed in binary32 (two roundings). Other arguments,
 * requirements and the workspace are those of mxfp4_gemm; with beta == 0 and FP32 output it runs
 * the same kernels as mxfp4_gemm.
 */
mxfp4_status_t mxfp4_gemm_ex(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                             const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs,
                             int64_t M, int64_t N, int64_t K, float alpha, float beta, void *c,
                             mxfp4_out_dtype_t c_dtype, int64_t ldc, mxfp4_layout_t layout,
                             void *workspace, size_t ws_bytes, void *stream);

/* Workspace bytes that let mxfp4_gemm split the contraction of an M x N x K product (0 when the
 * product is not split; also 0 for invalid sizes). */
size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* One product of a grouped launch: its operands (device, as for mxfp4_gemm) and its output. */
typedef struct {
    const uint8_t *aq, *as, *bq, *bs;
    float *c;
} mxfp4_gemm_item_t;

#define MXFP4_GEMM_GROUP_MAX 8

/*
 * mxfp4_gemm_grouped -- up to MXFP4_GEMM_GROUP_MAX products of one shape in one launch.
 *
 * Defined by: the product of mxfp4_gemm (Methodology section), for each item i:
 *   items[i].c = alpha * A_i B_i^T,  A_i = (items[i].aq, items[i].as), B_i = (items[i].bq, items[i].bs).
 * It serves the layer's products that have too few output tiles to fill the chip on their own
 * (the key and value projections of an attention block: one input, two weights of the same
 * shape): their tiles share one grid, so each output is the one mxfp4_gemm writes, bit for bit.
 *   items    host array of count entries, read before the call returns; every pointer as
 *            mxfp4_gemm requires it; the outputs must not overlap one another.
 *   count    0 .. MXFP4_GEMM_GROUP_MAX (0: nothing to do).
 * M, N, K, the leading dimensions, alpha and the layout apply to every item, with mxfp4_gemm's
 * requirements. No workspace: the contraction is never split. Row-major operands whose K is not
 * a multiple of 512 take the row kernel, one grid layer per item, still in one launch.
 * Errors: MXFP4_ERR_ARG for count out of range or overlapping outputs; otherwise those of
 * mxfp4_gemm, for the first item that fails them (nothing is launched then).
 */
mxfp4_status_t mxfp4_gemm_grouped(const mxfp4_gemm_item_t *items, int count, int64_t lda, int64_t ldas,
                                  int64_t ldb, int64_t ldbs, int64_t M, int64_t N, int64_t K, float alpha,
                                  int64_t ldc, mxfp4_layout_t layout, void *stream);

/* Per-operand configuration of one linear-layer GEMM. */
typedef struct {
    int hadamard;              /* 0, 16 or 32 (| MXFP4_RHT, | MXFP4_ORTHONORMAL): rotation along
                                  the contraction axis */
    mxfp4_rounding_t rnd_a;    /* rounding of the first operand (X, dY, dY^T) */
    mxfp4_rounding_t rnd_b;    /* rounding of the second operand (W, W^T, X^T) */
    uint64_t seed;             /* Philox key for stochastic rounding; stream 0 = first operand,
                                  stream 1 = second operand */
} mxfp4_linear_cfg_t;

/*
 * Workspace (device bytes) the linear calls need for the two quantized operands of `pass` at
 * X[M][K], W[N][K], dY[M][N] (tiled when the contraction is a multiple of 512), plus the split-K
 * partials of the product when it is split. Returns 0 for invalid sizes.
 */
size_t mxfp4_linear_workspace_bytes(mxfp4_pass_t pass, int64_t M, int64_t K, int64_t N);

/*
 * The three GEMMs of a linear layer Y = X W^T (Methodology section: Fprop, Dgrad, Wgrad), each
 * operand rotated along the GEMM's contraction axis and quantized to MXFP4, then multiplied on
 * the FP4 matrix cores with FP32 accumulation; alpha = 1/h is applied in the epilogue.
 *   fprop: y[M][N]  = X[M][K] . W[N][K]^T      (both quantized along K)
 *   dgrad: dx[M][K] = dY[M][N] . W[N][K]       (dY along N; W along N, i.e. transposed)
 *   wgrad: dw[N][K] = dY[M][N]^T . X[M][K]     (both along the token axis M, transposed)
 * Inputs are bf16, dense row-major (leading dimension = row length), 16-byte aligned; outputs
 * FP32 dense row-major. ws is a device buffer of at least mxfp4_linear_workspace_bytes() bytes,
 * 256-byte aligned, used only during the enqueued work (do not reuse it before it finishes).
 * The contraction length and every quantized length must be multiples of 32:
 * fprop K, dgrad N, wgrad M.
 */
mxfp4_status_t mxfp4_linear_fprop(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *y, void *stream);
mxfp4_status_t mxfp4_linear_dgrad(const void *dy_bf16, const void *w_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *dx, void *stream);
mxfp4_status_t mxfp4_linear_wgrad(const void *dy_bf16, const void *x_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *dw, void *stream);

/*
 * One training step of the linear layer, split where a training loop splits it: the forward
 * call needs X and W, the backward call dY. Each of X, W and dY is read and quantized ONCE, along
 * both of its axes (the one-pass quantizer of mxfp4_quantize_dual), instead of once per GEMM:
 *   mxfp4_linear_forward : X along K (Fprop) and along M (Wgrad), W along K (Fprop) and along N
 *                          (Dgrad); writes y[M][N] = Fprop and keeps the four quantizations in ws;
 *   mxfp4_linear_backward: dY along N (Dgrad) and along M (Wgrad); writes dx[M][K] = Dgrad and
 *                          dw[N][K] = Wgrad from the operands the forward call left in ws.
 * Roundings are per product, for both of its operands; Philox streams and keys are those of the
 * separate calls (stream 0 = first operand, 1 = second, key = seed), so y, dx and dw are
 * bitwise those of mxfp4_linear_fprop / _dgrad / _wgrad with cfg {hadamard, r, r, seed} and
 * r = fprop, dgrad, wgrad respectively.
 * Requirements: M, K and N are all contraction lengths here, so each must be a multiple of 32.
 * Inputs bf16 dense row-major, 16-byte aligned; outputs FP32 dense row-major, 4-byte aligned.
 * ws: at least mxfp4_linear_step_workspace_bytes(M, K, N) device bytes, 256-byte aligned; the
 * backward call must get the same ws, unchanged since the forward call of the same step (calls
 * on one stream are ordered; across streams the caller orders them). Errors as elsewhere:
 * MXFP4_ERR_WORKSPACE for a short ws, nothing launched on any argument error.
 */
typedef struct {
    int hadamard;              /* as in mxfp4_linear_cfg_t */
    mxfp4_rounding_t fprop;    /* X along K and W along K */
    mxfp4_rounding_t dgrad;    /* dY along N and W along N */
    mxfp4_rounding_t wgrad;    /* dY along M and X along M */
    uint64_t seed;             /* Philox key of every stochastic rounding of the step */
} mxfp4_step_cfg_t;

size_t mxfp4_linear_step_workspace_bytes(int64_t M, int64_t K, int64_t N);
mxfp4_status_t mxfp4_linear_forward(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                    int64_t N, const mxfp4_step_cfg_t *cfg, void *ws,
                                    size_t ws_bytes, float *y, void *stream);
mxfp4_status_t mxfp4_linear_backward(const void *dy_bf16, int64_t M, int64_t K, int64_t N,
                                     const mxfp4_step_cfg_t *cfg, void *ws, size_t ws_bytes,
                                     float *dx, float *dw, void *stream);

/*
 * mxfp4_linear_fprop without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, rules and result as mxfp4_linear_fprop (bitwise), except that the workspace is the
 * library's own device array of MXFP4_NOALLOC_SCRATCH_BYTES bytes: one per GPU the library runs
 * on, held until the process ends, looked up on the first call on each device. The call allocates
 * nothing. Products whose mxfp4_linear_workspace_bytes(MXFP4_FPROP, M, K, N) exceeds the array
 * return MXFP4_ERR_WORKSPACE before anything is launched (the Llama-3.1-8B QKV Fprop at 8192
 * tokens needs 30 MB; the down projection's Fprop, 94 MB, is refused). Every call on one GPU
 * shares its array: calls whose work overlaps on that GPU (other streams, other threads) race;
 * calls ordered on one stream do not.
 */
#define MXFP4_NOALLOC_SCRATCH_BYTES (64u << 20)
mxfp4_status_t mxfp4_linear_fprop_noalloc(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                          int64_t N, const mxfp4_linear_cfg_t *cfg, float *y, void *stream);

/* Static, NUL-terminated description of a status code. */
const char *mxfp4_status_string(mxfp4_status_t status);

/* MXFP4_ABI_VERSION of the built library. */
int mxfp4_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MXFP4_H_ */

// C-ABI entry points: argument validation, workspace carve-up and kernel dispatch.
// Every argument check happens before the first HIP call, so an invalid call launches nothing,
// touches no output and needs no device.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>

#include "../../include/mxfp4.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxBlocks = (int64_t)1 << 30;  // 32-element blocks per quantize launch
constexpr int64_t kMaxDim = ((int64_t)1 << 31) - 1;

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

mxfp4_status_t check_device()
{
    // gfx950 check, cached per device ordinal: 0 = unknown, 1 = gfx950, 2 = other
    static std::atomic<int> cache[64];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MXFP4_ERR_DEVICE;
    if (dev < 64) {
        const int known = cache[dev].load(std::memory_order_relaxed);
        if (known) return known == 1 ? MXFP4_OK : MXFP4_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MXFP4_ERR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? MXFP4_OK : MXFP4_ERR_DEVICE;
}

mxfp4_status_t from_hip(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_LAUNCH; }

// Validation of one quantize call; also used by the linear entry points.
static_assert(MXFP4_RHT == mx::kRandomizedHadamard, "randomized-Hadamard flag");
static_assert(MXFP4_ORTHONORMAL == mx::kOrthonormal, "orthonormal-rotation flag");

// rounding: MXFP4_RNE or MXFP4_SR_PHILOX, optionally with MXFP4_SCALE_NOCLIP
bool valid_rounding(int rounding)
{
    const int r = rounding & ~MXFP4_SCALE_NOCLIP;
    return r == MXFP4_RNE || r == MXFP4_SR_PHILOX;
}
bool is_sr(int rounding) { return (rounding & ~MXFP4_SCALE_NOCLIP) == MXFP4_SR_PHILOX; }
bool is_noclip(int rounding) { return (rounding & MXFP4_SCALE_NOCLIP) != 0; }

// hadamard: 0, 16 or 32, or 16 / 32 with MXFP4_RHT and / or MXFP4_ORTHONORMAL
bool valid_rotation(int hadamard)
{
    const int flags = MXFP4_RHT | MXFP4_ORTHONORMAL;
    const int h = hadamard & ~flags;
    if (h != 0 && h != 16 && h != 32) return false;
    return !((hadamard & flags) && h == 0);
}

mxfp4_status_t check_quantize(const void *x, mxfp4_dtype_t dtype, int64_t rows, int64_t cols,
                              int64_t ldx, int axis, int hadamard, mxfp4_rounding_t rounding,
                              mxfp4_layout_t layout, const uint8_t *q, int64_t ldq,
                              const uint8_t *scales, int64_t lds)
{
    if (layout != MXFP4_LAYOUT_ROWS && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_ARG;
    const bool tiled = layout == MXFP4_LAYOUT_TILED;
    if (dtype != MXFP4_IN_BF16 && dtype != MXFP4_IN_F32) return MXFP4_ERR_ARG;
    if (axis != 0 && axis != 1) return MXFP4_ERR_ARG;
    if (!valid_rotation(hadamard)) return MXFP4_ERR_ARG;
    if (!valid_rounding(rounding)) return MXFP4_ERR_ARG;
    if (rows < 0 || cols < 0 || rows > kMaxDim || cols > kMaxDim) return MXFP4_ERR_SHAPE;
    const int64_t L = axis ? cols : rows;
    const int64_t outer = axis ? rows : cols;
    if (L % (tiled ? 512 : 32) != 0) return MXFP4_ERR_SHAPE;
    if (outer > 0 && L / 32 > 0 && outer > kMaxBlocks / (L / 32)) return MXFP4_ERR_SHAPE;
    if (ldx < cols || ldx < 1) return MXFP4_ERR_ARG;
    if (!tiled && (ldq < L / 2 || lds < L / 32)) return MXFP4_ERR_ARG;
    if (rows == 0 || cols == 0) return MXFP4_OK;
    if (!x || !q || !scales) return MXFP4_ERR_NULL;
    const int64_t esize = dtype == MXFP4_IN_F32 ? 4 : 2;
    if (!aligned(x, 16) || (ldx * esize) % 16 != 0) return MXFP4_ERR_ALIGN;
    if (!aligned(q, 16)) return MXFP4_ERR_ALIGN;
    if (tiled ? !aligned(scales, 16) : ldq % 16 != 0) return MXFP4_ERR_ALIGN;
    return MXFP4_OK;
}

int64_t pad256(int64_t v) { return (v + 255) / 256 * 256; }

mxfp4_status_t check_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                          const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs,
                          int64_t M, int64_t N, int64_t K, const void *c, int64_t ldc,
                          mxfp4_layout_t layout, size_t c_elem = 4)
{
    if (layout != MXFP4_LAYOUT_ROWS && layout != MXFP4_LAYOUT_TILED) return MXFP4_ERR_ARG;
    const bool tiled = layout == MXFP4_LAYOUT_TILED;
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return MXFP4_ERR_SHAPE;
    if (K % (tiled ? 512 : 32) != 0) return MXFP4_ERR_SHAPE;
    // tiled operands are addressed with 32-bit byte offsets
    if (tiled && (pad256(M) * (K / 2) > (int64_t)UINT32_MAX || pad256(N) * (K / 2) > (int64_t)UINT32_MAX))
        return MXFP4_ERR_SHAPE;
    if (ldc < N || ldc < 1) return MXFP4_ERR_ARG;
    if (!tiled && (lda < K / 2 || ldb < K / 2 || ldas < K / 32 || ldbs < K / 32)) return MXFP4_ERR_ARG;
    if (M == 0 || N == 0) return MXFP4_OK;
    if (!c) return MXFP4_ERR_NULL;
    if (K > 0 && (!aq || !as || !bq || !bs)) return MXFP4_ERR_NULL;
    if (!aligned(aq, 16) || !aligned(bq, 16)) return MXFP4_ERR_ALIGN;
    if (tiled ? (!aligned(as, 16) || !aligned(bs, 16)) : (lda % 16 != 0 || ldb % 16 != 0))
        return MXFP4_ERR_ALIGN;
    if (!aligned(c, c_elem)) return MXFP4_ERR_ALIGN;
    return MXFP4_OK;
}

// Workspace layout of one linear call: A codes | A scales | B codes | B scales, each 256-aligned.
// Contractions that are multiples of 512 use the tiled layout (rows padded to 256).
struct OperandSpace {
    int64_t outer, L;
    bool tiled() const { return L > 0 && L % 512 == 0; }
    int64_t rows() const { return tiled() ? pad256(outer) : outer; }
    size_t codes() const { return (size_t)rows() * (size_t)(L / 2); }
    size_t scales() const { return (size_t)rows() * (size_t)(L / 32); }
};

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

size_t layout_bytes(const OperandSpace &a, const OperandSpace &b)
{
    return round256(a.codes()) + round256(a.scales()) + round256(b.codes()) + round256(b.scales());
}

// bytes of the operand part plus the split-K partials of the (out_rows x out_cols x kc) product
size_t linear_bytes(const OperandSpace &a, const OperandSpace &b, int64_t out_rows, int64_t out_cols, int64_t kc)
{
    return layout_bytes(a, b) + round256(mx::gemm_workspace_bytes(out_rows, out_cols, kc));
}

bool pass_operands(mxfp4_pass_t pass, int64_t M, int64_t K, int64_t N, OperandSpace *a, OperandSpace *b)
{
    switch (pass) {
    case MXFP4_FPROP: *a = {M, K}; *b = {N, K}; return true;   // X along K, W along K
    case MXFP4_DGRAD: *a = {M, N}; *b = {K, N}; return true;   // dY along N, W^T along N
    case MXFP4_WGRAD: *a = {N, M}; *b = {K, M}; return true;   // dY^T along M, X^T along M
    default: break;
    }
    return false;
}

struct LinearSpec {
    const void *a_src; int64_t a_rows, a_cols; int a_axis;  // first operand tensor and its axis
    const void *b_src; int64_t b_rows, b_cols; int b_axis;
    int64_t out_rows, out_cols, kc;                          // GEMM output and contraction
};

mxfp4_status_t run_linear(const LinearSpec &sp, mxfp4_pass_t pass, int64_t M, int64_t K, int64_t N,
                          const mxfp4_linear_cfg_t *cfg, void *ws, size_t ws_bytes, float *out,
                          void *stream)
{
    if (!cfg) return MXFP4_ERR_NULL;
    if (M < 0 || K < 0 || N < 0 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return MXFP4_ERR_SHAPE;
    if (!valid_rotation(cfg->hadamard)) return MXFP4_ERR_ARG;
    if (!valid_rounding(cfg->rnd_a) || !valid_rounding(cfg->rnd_b)) return MXFP4_ERR_ARG;
    if (sp.kc % 32 != 0) return MXFP4_ERR_SHAPE;
    OperandSpace a, b;
    pass_operands(pass, M, K, N, &a, &b);
    if (a.outer > 0 && a.L / 32 > 0 && (a.outer > kMaxBlocks / (a.L / 32) || b.outer > kMaxBlocks / (a.L / 32)))
        return MXFP4_ERR_SHAPE;
    const bool tiled = a.tiled();
    if (tiled && (a.codes() > UINT32_MAX || b.codes() > UINT32_MAX)) return MXFP4_ERR_SHAPE;
    if (sp.out_rows == 0 || sp.out_cols == 0) return MXFP4_OK;
    if (!out) return MXFP4_ERR_NULL;
    if (!aligned(out, 4)) return MXFP4_ERR_ALIGN;
    // H H^T = h I, also with the randomized sign diagonal (D D^T = I); the orthonormal rotation
    // (H / sqrt(h)) (H / sqrt(h))^T = I needs no factor
    const int h = cfg->hadamard & ~(MXFP4_RHT | MXFP4_ORTHONORMAL);
    const float alpha = (cfg->hadamard & MXFP4_ORTHONORMAL) || h == 0 ? 1.0f : 1.0f / (float)h;
    if (sp.kc == 0) {
        // empty contraction: the product is all zeros
        if (mxfp4_status_t st = check_device()) return st;
        return from_hip(mx::launch_empty_product(out, false, sp.out_rows, sp.out_cols, sp.out_cols, 0.0f,
                                                 (hipStream_t)stream));
    }
    if (!sp.a_src || !sp.b_src) return MXFP4_ERR_NULL;
    if (!aligned(sp.a_src, 16) || !aligned(sp.b_src, 16)) return MXFP4_ERR_ALIGN;
    if ((sp.a_cols * 2) % 16 != 0 || (sp.b_cols * 2) % 16 != 0) return MXFP4_ERR_ALIGN;
    const size_t need = linear_bytes(a, b, sp.out_rows, sp.out_cols, sp.kc);
    if (!ws || ws_bytes < need) return MXFP4_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return MXFP4_ERR_ALIGN;
    if (mxfp4_status_t st = check_device()) return st;

    uint8_t *p = static_cast<uint8_t *>(ws);
    uint8_t *aq = p;
    uint8_t *as = aq + round256(a.codes());
    uint8_t *bq = as + round256(a.scales());
    uint8_t *bs = bq + round256(b.codes());
    hipStream_t s = (hipStream_t)stream;
    auto quant = [&](const void *src, int64_t rows, int64_t cols, int axis, mxfp4_rounding_t rnd,
                     uint32_t sid, uint8_t *q, uint8_t *sc, int64_t L) {
        if (axis == 1)
            return mx::launch_quantize_rows(src, false, rows, cols, cols, cfg->hadamard, is_sr(rnd),
                                            is_noclip(rnd), cfg->seed, sid, tiled, q, L / 2, sc, L / 32, s);
        return mx::launch_quantize_cols(src, false, rows, cols, cols, cfg->hadamard, is_sr(rnd),
                                        is_noclip(rnd), cfg->seed, sid, tiled, q, L / 2, sc, L / 32, s);
    };
    hipError_t e = quant(sp.a_src, sp.a_rows, sp.a_cols, sp.a_axis, cfg->rnd_a, 0u, aq, as, a.L);
    if (e == hipSuccess) e = quant(sp.b_src, sp.b_rows, sp.b_cols, sp.b_axis, cfg->rnd_b, 1u, bq, bs, b.L);
    if (e == hipSuccess)
        e = mx::launch_gemm(aq, a.L / 2, as, a.L / 32, bq, b.L / 2, bs, b.L / 32, sp.out_rows,
                            sp.out_cols, sp.kc, alpha, 0.0f, out, false, sp.out_cols, tiled,
                            p + layout_bytes(a, b), ws_bytes - layout_bytes(a, b), s);
    return from_hip(e);
}

// ---------------------------------------------------------------- training step ----------
// Workspace of one step: X, W and dY quantized along both axes, each laid out as the separate
// linear calls lay it out (tiled when its quantized length is a multiple of 512), then the
// split-K partials of the largest of the three products (the products run one after another).
enum { kXr, kWr, kXc, kWc, kDYr, kDYc, kStepOperands };

struct StepSpace {
    OperandSpace op[kStepOperands];
    size_t off[kStepOperands];  // codes at off, scales at off + round256(codes)
    size_t splitk_off, total;
};

StepSpace step_space(int64_t M, int64_t K, int64_t N)
{
    StepSpace sp;
    sp.op[kXr] = {M, K};   // X along K: Fprop A
    sp.op[kWr] = {N, K};   // W along K: Fprop B
    sp.op[kXc] = {K, M};   // X along M: Wgrad B
    sp.op[kWc] = {K, N};   // W along N: Dgrad B
    sp.op[kDYr] = {M, N};  // dY along N: Dgrad A
    sp.op[kDYc] = {N, M};  // dY along M: Wgrad A
    size_t o = 0;
    for (int i = 0; i < kStepOperands; ++i) {
        sp.off[i] = o;
        o += round256(sp.op[i].codes()) + round256(sp.op[i].scales());
    }
    sp.splitk_off = o;
    size_t sk = mx::gemm_workspace_bytes(M, N, K);
    sk = std::max(sk, mx::gemm_workspace_bytes(M, K, N));
    sk = std::max(sk, mx::gemm_workspace_bytes(N, K, M));
    sp.total = o + round256(sk);
    return sp;
}

mxfp4_status_t check_step(int64_t M, int64_t K, int64_t N, const mxfp4_step_cfg_t *cfg, const void *ws,
                          size_t ws_bytes, StepSpace *sp)
{
    if (!cfg) return MXFP4_ERR_NULL;
    if (M < 0 || K < 0 || N < 0 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return MXFP4_ERR_SHAPE;
    if (M % 32 != 0 || K % 32 != 0 || N % 32 != 0) return MXFP4_ERR_SHAPE;
    if (!valid_rotation(cfg->hadamard)) return MXFP4_ERR_ARG;
    if (!valid_rounding(cfg->fprop) || !valid_rounding(cfg->dgrad) || !valid_rounding(cfg->wgrad))
        return MXFP4_ERR_ARG;
    *sp = step_space(M, K, N);
    for (const OperandSpace &o : sp->op) {
        if (o.L / 32 > 0 && o.outer > kMaxBlocks / (o.L / 32)) return MXFP4_ERR_SHAPE;
        if (o.tiled() && o.codes() > UINT32_MAX) return MXFP4_ERR_SHAPE;
    }
    if (ws_bytes < sp->total || (sp->total > 0 && !ws)) return MXFP4_ERR_WORKSPACE;
    if (ws && !aligned(ws, 256)) return MXFP4_ERR_ALIGN;
    return MXFP4_OK;
}

float step_alpha(int hadamard)
{
    const int h = hadamard & ~(MXFP4_RHT | MXFP4_ORTHONORMAL);
    return (hadamard & MXFP4_ORTHONORMAL) || h == 0 ? 1.0f : 1.0f / (float)h;
}

// one output of a step's dual quantization, into the workspace
mx::QuantOut step_out(const StepSpace &sp, int which, uint8_t *ws, mxfp4_rounding_t rnd, uint64_t seed,
                      uint32_t stream_id)
{
    const OperandSpace &o = sp.op[which];
    uint8_t *q = ws + sp.off[which];
    return mx::QuantOut{is_sr(rnd), is_noclip(rnd), seed, stream_id, o.tiled(), q, o.L / 2,
                        q + round256(o.codes()), o.L / 32};
}

// out[rows][cols] = alpha A B^T over the contraction of operands a, b of the workspace (zero for
// an empty contraction)
hipError_t step_gemm(const StepSpace &sp, int a, int b, uint8_t *ws, size_t ws_bytes, int64_t rows, int64_t cols,
                     float alpha, float *out, hipStream_t s)
{
    const OperandSpace &oa = sp.op[a], &ob = sp.op[b];
    if (rows == 0 || cols == 0) return hipSuccess;
    if (oa.L == 0) return mx::launch_empty_product(out, false, rows, cols, cols, 0.0f, s);
    const uint8_t *aq = ws + sp.off[a], *bq = ws + sp.off[b];
    return mx::launch_gemm(aq, oa.L / 2, aq + round256(oa.codes()), oa.L / 32, bq, ob.L / 2,
                           bq + round256(ob.codes()), ob.L / 32, rows, cols, oa.L, alpha, 0.0f, out, false, cols,
                           oa.tiled(), ws + sp.splitk_off, ws_bytes - sp.splitk_off, s);
}

bool input_ok(const void *p) { return p != nullptr && aligned(p, 16); }

}  // namespace

extern "C" {

mxfp4_status_t mxfp4_quantize(const void *x, mxfp4_dtype_t dtype, int64_t rows, int64_t cols,
                              int64_t ldx, int axis, int hadamard, mxfp4_rounding_t rounding,
                              uint64_t seed, uint32_t stream_id, mxfp4_layout_t layout, uint8_t *q,
                              int64_t ldq, uint8_t *scales, int64_t lds, void *stream)
{
    mxfp4_status_t st = check_quantize(x, dtype, rows, cols, ldx, axis, hadamard, rounding, layout,
                                       q, ldq, scales, lds);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    const bool f32 = dtype == MXFP4_IN_F32;
    const bool sr = is_sr(rounding), noclip = is_noclip(rounding);
    const bool tiled = layout == MXFP4_LAYOUT_TILED;
    hipError_t e = axis == 1
        ? mx::launch_quantize_rows(x, f32, rows, cols, ldx, hadamard, sr, noclip, seed, stream_id, tiled, q,
                                   ldq, scales, lds, (hipStream_t)stream)
        : mx::launch_quantize_cols(x, f32, rows, cols, ldx, hadamard, sr, noclip, seed, stream_id, tiled, q,
                                   ldq, scales, lds, (hipStream_t)stream);
    return from_hip(e);
}

mxfp4_status_t mxfp4_quantize_dual(const void *x, mxfp4_dtype_t dtype, int64_t rows, int64_t cols,
                                   int64_t ldx, int hadamard, const mxfp4_quant_out_t *out_axis1,
                                   const mxfp4_quant_out_t *out_axis0, void *stream)
{
    if (!out_axis1 || !out_axis0) return MXFP4_ERR_NULL;
    const mxfp4_quant_out_t &a = *out_axis1, &b = *out_axis0;
    mxfp4_status_t st = check_quantize(x, dtype, rows, cols, ldx, 1, hadamard, a.rounding, a.layout,
                                       a.q, a.ldq, a.scales, a.lds);
    if (st == MXFP4_OK)
        st = check_quantize(x, dtype, rows, cols, ldx, 0, hadamard, b.rounding, b.layout, b.q, b.ldq,
                            b.scales, b.lds);
    if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    const auto conv = [](const mxfp4_quant_out_t &o) {
        return mx::QuantOut{is_sr(o.rounding), is_noclip(o.rounding), o.seed, o.stream_id,
                            o.layout == MXFP4_LAYOUT_TILED, o.q, o.ldq, o.scales, o.lds};
    };
    return from_hip(mx::launch_quantize_dual(x, dtype == MXFP4_IN_F32, rows, cols, ldx, hadamard, conv(a),
                                             conv(b), (hipStream_t)stream));
}

static_assert(MXFP4_DUAL_GROUP_MAX == mx::kDualGroupMax, "grouped dual quantizer capacity");

mxfp4_status_t mxfp4_quantize_dual_grouped(const mxfp4_dual_item_t *items, int count, int hadamard,
                                           void *stream)
{
    if (count < 0 || count > MXFP4_DUAL_GROUP_MAX) return MXFP4_ERR_ARG;
    if (count == 0) return MXFP4_OK;
    if (!items) return MXFP4_ERR_NULL;
    mxfp4_status_t st;
    bool any = false;
    for (int i = 0; i < count; ++i) {
        const mxfp4_dual_item_t &it = items[i];
        if (it.dtype != items[0].dtype) return MXFP4_ERR_ARG;
        const mxfp4_quant_out_t &a = it.axis1, &b = it.axis0;
        if ((st = check_quantize(it.x, it.dtype, it.rows, it.cols, it.ldx, 1, hadamard, a.rounding, a.layout, a.q,
                                 a.ldq, a.scales, a.lds)) != MXFP4_OK)
            return st;
        if ((st = check_quantize(it.x, it.dtype, it.rows, it.cols, it.ldx, 0, hadamard, b.rounding, b.layout, b.q,
                                 b.ldq, b.scales, b.lds)) != MXFP4_OK)
            return st;
        any = any || (it.rows > 0 && it.cols > 0);
    }
    if (!any) return MXFP4_OK;
    if ((st = check_device()) != MXFP4_OK) return st;
    const auto conv = [](const mxfp4_quant_out_t &o) {
        return mx::QuantOut{is_sr(o.rounding), is_noclip(o.rounding), o.seed, o.stream_id,
                            o.layout == MXFP4_LAYOUT_TILED, o.q, o.ldq, o.scales, o.lds};
    };
    mx::DualInput in[MXFP4_DUAL_GROUP_MAX];
    for (int i = 0; i < count; ++i)
        in[i] = mx::DualInput{items[i].x, items[i].rows, items[i].cols, items[i].ldx, conv(items[i].axis1),
                              conv(items[i].axis0)};
    return from_hip(mx::launch_quantize_dual_grouped(in, count, items[0].dtype == MXFP4_IN_F32, hadamard,
                                                     (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                          const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs,
                          int64_t M, int64_t N, int64_t K, float alpha, float *c, int64_t ldc,
                          mxfp4_layout_t layout, void *workspace, size_t ws_bytes, void *stream)
{
    mxfp4_status_t st = check_gemm(aq, lda, as, ldas, bq, ldb, bs, ldbs, M, N, K, c, ldc, layout);
    if (st != MXFP4_OK || M == 0 || N == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    if (K == 0) {
        // empty contraction: the product is all zeros
        return from_hip(mx::launch_empty_product(c, false, M, N, ldc, 0.0f, (hipStream_t)stream));
    }
    return from_hip(mx::launch_gemm(aq, lda, as, ldas, bq, ldb, bs, ldbs, M, N, K, alpha, 0.0f, c, false, ldc,
                                    layout == MXFP4_LAYOUT_TILED, workspace, ws_bytes,
                                    (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm_ex(const uint8_t *aq, int64_t lda, const uint8_t *as, int64_t ldas,
                             const uint8_t *bq, int64_t ldb, const uint8_t *bs, int64_t ldbs,
                             int64_t M, int64_t N, int64_t K, float alpha, float beta, void *c,
                             mxfp4_out_dtype_t c_dtype, int64_t ldc, mxfp4_layout_t layout,
                             void *workspace, size_t ws_bytes, void *stream)
{
    if (c_dtype != MXFP4_OUT_F32 && c_dtype != MXFP4_OUT_BF16) return MXFP4_ERR_ARG;
    const bool bf16 = c_dtype == MXFP4_OUT_BF16;
    mxfp4_status_t st = check_gemm(aq, lda, as, ldas, bq, ldb, bs, ldbs, M, N, K, c, ldc, layout, bf16 ? 2 : 4);
    if (st != MXFP4_OK || M == 0 || N == 0) return st;
    if ((st = check_device()) != MXFP4_OK) return st;
    if (K == 0) return from_hip(mx::launch_empty_product(c, bf16, M, N, ldc, beta, (hipStream_t)stream));
    return from_hip(mx::launch_gemm(aq, lda, as, ldas, bq, ldb, bs, ldbs, M, N, K, alpha, beta, c, bf16, ldc,
                                    layout == MXFP4_LAYOUT_TILED, workspace, ws_bytes,
                                    (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm_grouped(const mxfp4_gemm_item_t *items, int count, int64_t lda, int64_t ldas,
                                  int64_t ldb, int64_t ldbs, int64_t M, int64_t N, int64_t K, float alpha,
                                  int64_t ldc, mxfp4_layout_t layout, void *stream)
{
    if (count < 0 || count > MXFP4_GEMM_GROUP_MAX) return MXFP4_ERR_ARG;
    if (count > 0 && !items) return MXFP4_ERR_NULL;
    mxfp4_status_t st;
    for (int i = 0; i < count; ++i) {
        const mxfp4_gemm_item_t &it = items[i];
        if ((st = check_gemm(it.aq, lda, it.as, ldas, it.bq, ldb, it.bs, ldbs, M, N, K, it.c, ldc, layout)) !=
            MXFP4_OK)
            return st;
    }
    if (count == 0 || M == 0 || N == 0) return MXFP4_OK;
    // the rows [c, c + (M - 1) ldc + N) of two outputs must not share an element
    const unsigned __int128 span = ((unsigned __int128)(M - 1) * (uint64_t)ldc + (uint64_t)N) * sizeof(float);
    for (int i = 0; i < count; ++i)
        for (int j = i + 1; j < count; ++j) {
            const unsigned __int128 a = (uintptr_t)items[i].c, b = (uintptr_t)items[j].c;
            if (a < b + span && b < a + span) return MXFP4_ERR_ARG;
        }
    if ((st = check_device()) != MXFP4_OK) return st;
    mx::GemmGroupItem grp[MXFP4_GEMM_GROUP_MAX];
    for (int i = 0; i < count; ++i) grp[i] = {items[i].aq, items[i].as, items[i].bq, items[i].bs, items[i].c};
    if (K == 0) {
        for (int i = 0; i < count; ++i) {
            const hipError_t e = mx::launch_empty_product(grp[i].c, false, M, N, ldc, 0.0f, (hipStream_t)stream);
            if (e != hipSuccess) return from_hip(e);
        }
        return MXFP4_OK;
    }
    return from_hip(mx::launch_gemm_grouped(grp, count, lda, ldas, ldb, ldbs, M, N, K, alpha, ldc,
                                            layout == MXFP4_LAYOUT_TILED, (hipStream_t)stream));
}

size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
    return mx::gemm_workspace_bytes(M, N, K);
}

mxfp4_status_t mxfp4_tiled_sizes(int64_t outer, int64_t L, size_t *codes_bytes, size_t *scales_bytes)
{
    if (!codes_bytes || !scales_bytes) return MXFP4_ERR_NULL;
    if (outer < 0 || L < 0 || outer > kMaxDim || L > kMaxDim || L % 512 != 0) return MXFP4_ERR_SHAPE;
    *codes_bytes = (size_t)pad256(outer) * (size_t)(L / 2);
    *scales_bytes = (size_t)pad256(outer) * (size_t)(L / 32);
    return MXFP4_OK;
}

size_t mxfp4_linear_workspace_bytes(mxfp4_pass_t pass, int64_t M, int64_t K, int64_t N)
{
    if (M < 0 || K < 0 || N < 0 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
    OperandSpace a, b;
    if (!pass_operands(pass, M, K, N, &a, &b)) return 0;
    // product shape of the pass: Fprop M x N (K), Dgrad M x K (N), Wgrad N x K (M)
    if (pass == MXFP4_FPROP) return linear_bytes(a, b, M, N, K);
    if (pass == MXFP4_DGRAD) return linear_bytes(a, b, M, K, N);
    return linear_bytes(a, b, N, K, M);
}

mxfp4_status_t mxfp4_linear_fprop(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *y, void *stream)
{
    LinearSpec sp{x_bf16, M, K, 1, w_bf16, N, K, 1, M, N, K};
    return run_linear(sp, MXFP4_FPROP, M, K, N, cfg, ws, ws_bytes, y, stream);
}

mxfp4_status_t mxfp4_linear_dgrad(const void *dy_bf16, const void *w_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *dx, void *stream)
{
    LinearSpec sp{dy_bf16, M, N, 1, w_bf16, N, K, 0, M, K, N};
    return run_linear(sp, MXFP4_DGRAD, M, K, N, cfg, ws, ws_bytes, dx, stream);
}

mxfp4_status_t mxfp4_linear_wgrad(const void *dy_bf16, const void *x_bf16, int64_t M, int64_t K,
                                  int64_t N, const mxfp4_linear_cfg_t *cfg, void *ws,
                                  size_t ws_bytes, float *dw, void *stream)
{
    LinearSpec sp{dy_bf16, M, N, 0, x_bf16, M, K, 0, N, K, M};
    return run_linear(sp, MXFP4_WGRAD, M, K, N, cfg, ws, ws_bytes, dw, stream);
}

size_t mxfp4_linear_step_workspace_bytes(int64_t M, int64_t K, int64_t N)
{
    if (M < 0 || K < 0 || N < 0 || M > kMaxDim || K > kMaxDim || N > kMaxDim) return 0;
    return step_space(M, K, N).total;
}

mxfp4_status_t mxfp4_linear_forward(const void *x_bf16, const void *w_bf16, int64_t M, int64_t K,
                                    int64_t N, const mxfp4_step_cfg_t *cfg, void *ws,
                                    size_t ws_bytes, float *y, void *stream)
{
    StepSpace sp;
    if (mxfp4_status_t st = check_step(M, K, N, cfg, ws, ws_bytes, &sp)) return st;
    const bool need_x = M > 0 && K > 0, need_w = N > 0 && K > 0, need_y = M > 0 && N > 0;
    if ((need_x && !x_bf16) || (need_w && !w_bf16) || (need_y && !y)) return MXFP4_ERR_NULL;
    if ((need_x && !input_ok(x_bf16)) || (need_w && !input_ok(w_bf16)) || (need_y && !aligned(y, 4)))
        return MXFP4_ERR_ALIGN;
    if (!need_x && !need_w && !need_y) return MXFP4_OK;
    if (mxfp4_status_t st = check_device()) return st;
    uint8_t *p = static_cast<uint8_t *>(ws);
    hipStream_t s = (hipStream_t)stream;
    const uint64_t seed = cfg->seed;
    hipError_t e = hipSuccess;
    // X: along K for Fprop (first operand, stream 0), along M for Wgrad (second operand, stream 1)
    if (need_x)
        e = mx::launch_quantize_dual(x_bf16, false, M, K, K, cfg->hadamard, step_out(sp, kXr, p, cfg->fprop, seed, 0u),
                                     step_out(sp, kXc, p, cfg->wgrad, seed, 1u), s);
    // W: along K for Fprop, along N for Dgrad (second operand of both, stream 1)
    if (e == hipSuccess && need_w)
        e = mx::launch_quantize_dual(w_bf16, false, N, K, K, cfg->hadamard, step_out(sp, kWr, p, cfg->fprop, seed, 1u),
                                     step_out(sp, kWc, p, cfg->dgrad, seed, 1u), s);
    if (e == hipSuccess) e = step_gemm(sp, kXr, kWr, p, ws_bytes, M, N, step_alpha(cfg->hadamard), y, s);
    return from_hip(e);
}

mxfp4_status_t mxfp4_linear_backward(const void *dy_bf16, int64_t M, int64_t K, int64_t N,
                                     const mxfp4_step_cfg_t *cfg, void *ws, size_t ws_bytes,
                                     float *dx, float *dw, void *stream)
{
    StepSpace sp;
    if (mxfp4_status_t st = check_step(M, K, N, cfg, ws, ws_bytes, &sp)) return st;
    const bool need_dy = M > 0 && N > 0, need_dx = M > 0 && K > 0, need_dw = N > 0 && K > 0;
    if ((need_dy && !dy_bf16) || (need_dx && !dx) || (need_dw && !dw)) return MXFP4_ERR_NULL;
    if ((need_dy && !input_ok(dy_bf16)) || (need_dx && !aligned(dx, 4)) || (need_dw && !aligned(dw, 4)))
        return MXFP4_ERR_ALIGN;
    if (!need_dy && !need_dx && !need_dw) return MXFP4_OK;
    if (mxfp4_status_t st = check_device()) return st;
    uint8_t *p = static_cast<uint8_t *>(ws);
    hipStream_t s = (hipStream_t)stream;
    const float alpha = step_alpha(cfg->hadamard);
    hipError_t e = hipSuccess;
    // dY: along N for Dgrad, along M for Wgrad (first operand of both, stream 0)
    if (need_dy)
        e = mx::launch_quantize_dual(dy_bf16, false, M, N, N, cfg->hadamard,
                                     step_out(sp, kDYr, p, cfg->dgrad, cfg->seed, 0u),
                                     step_out(sp, kDYc, p, cfg->wgrad, cfg->seed, 0u), s);
    if (e == hipSuccess) e = step_gemm(sp, kDYr, kWc, p, ws_bytes, M, K, alpha, dx, s);
    if (e == hipSuccess) e = step_gemm(sp, kDYc, kXc, p, ws_bytes, N, K, alpha, dw, s);
    return from_hip(e);
}

const char *mxfp4_status_string(mxfp4_status_t status)
{
    switch (status) {
    case MXFP4_OK: return "ok";
    case MXFP4_ERR_NULL: return "a required pointer is NULL";
    case MXFP4_ERR_SHAPE: return "invalid shape (negative size, length not a multiple of 32, or too large)";
    case MXFP4_ERR_ARG: return "invalid argument (enum, hadamard size or leading dimension)";
    case MXFP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case MXFP4_ERR_WORKSPACE: return "workspace missing or too small";
    case MXFP4_ERR_DEVICE: return "no current gfx950 device";
    case MXFP4_ERR_LAUNCH: return "kernel launch failed";
    default: break;
    }
    return "unknown status";
}

int mxfp4_abi_version(void) { return MXFP4_ABI_VERSION; }

}  // extern "C"

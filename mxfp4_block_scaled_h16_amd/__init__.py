"""MXFP4 + block-Hadamard linear-layer GEMMs on AMD MI355X (gfx950).

Thin ctypes binding over ``libmxfp4.so`` (C ABI declared in ``include/mxfp4.h``). Every step of
the hot path runs in the library's HIP kernels; this module only marshals arguments. PyTorch
provides device memory (tensors) and the stream (the current HIP stream).

The three GEMMs are those of the gist.science summary of "MXFP4 LLM pretraining", section 방법론
(Methodology): Fprop Y = X W^T, Dgrad dX = dY W, Wgrad dW = dY^T X, each operand rotated by a
deterministic block Hadamard (H16 / H32) along the GEMM's contraction axis and quantized to MXFP4.
"""
import ctypes
import os

import torch  # imported first: the library binds to the HIP runtime torch has loaded

__all__ = [
    "Mxfp4Error", "RHT", "ORTHO", "SCALE_NOCLIP", "quantize", "quantize_dual", "gemm", "linear_fprop",
    "linear_dgrad", "linear_wgrad", "linear_forward", "linear_backward", "step_workspace_bytes", "workspace_bytes", "library_path", "lib", "RNE", "SR", "FPROP", "DGRAD", "WGRAD", "ROWS", "TILED",
    "tiled_sizes", "gemm_workspace_bytes", "linear_fprop_noalloc", "NOALLOC_SCRATCH_BYTES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp4.so")

RNE, SR = 0, 1
FPROP, DGRAD, WGRAD = 0, 1, 2
ROWS, TILED = 0, 1
BF16, F32 = 0, 1
RHT = 0x100  # OR into hadamard (16 or 32): randomized Hadamard, signs keyed by the seed
ORTHO = 0x200  # OR into hadamard (16 or 32): orthonormal rotation H_h / sqrt(h) (GEMM alpha 1)
SCALE_NOCLIP = 0x10  # OR into rounding: the smallest scale that maps the block maximum to <= 6

_lib = None


class Mxfp4Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, _status_string(status), status))


class QuantOut(ctypes.Structure):
    """mxfp4_quant_out_t: one output of mxfp4_quantize_dual."""
    _fields_ = [("rounding", ctypes.c_int), ("seed", ctypes.c_uint64), ("stream_id", ctypes.c_uint32),
                ("layout", ctypes.c_int), ("q", ctypes.c_void_p), ("ldq", ctypes.c_int64),
                ("scales", ctypes.c_void_p), ("lds", ctypes.c_int64)]


class DualItem(ctypes.Structure):
    """mxfp4_dual_item_t: one tensor of mxfp4_quantize_dual_grouped."""
    _fields_ = [("x", ctypes.c_void_p), ("dtype", ctypes.c_int), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("ldx", ctypes.c_int64), ("axis1", QuantOut), ("axis0", QuantOut)]


class GemmItem(ctypes.Structure):
    """mxfp4_gemm_item_t: one product of mxfp4_gemm_grouped."""
    _fields_ = [("aq", ctypes.c_void_p), ("as_", ctypes.c_void_p), ("bq", ctypes.c_void_p),
                ("bs", ctypes.c_void_p), ("c", ctypes.c_void_p)]


class LinearCfg(ctypes.Structure):
    _fields_ = [("hadamard", ctypes.c_int), ("rnd_a", ctypes.c_int), ("rnd_b", ctypes.c_int),
                ("seed", ctypes.c_uint64)]


class StepCfg(ctypes.Structure):
    """mxfp4_step_cfg_t: rotation, per-product roundings and the Philox key of a training step."""
    _fields_ = [("hadamard", ctypes.c_int), ("fprop", ctypes.c_int), ("dgrad", ctypes.c_int),
                ("wgrad", ctypes.c_int), ("seed", ctypes.c_uint64)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded C library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("%s is missing: build it with `python -m mxfp4_block_scaled_h16_amd.build` "
                          "(or __graft_entry__.build())" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    i64, u64, u32, vp, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    L.mxfp4_quantize.argtypes = [vp, ci, i64, i64, i64, ci, ci, ci, u64, u32, ci, vp, i64, vp, i64, vp]
    L.mxfp4_quantize.restype = ci
    L.mxfp4_quantize_dual.argtypes = [vp, ci, i64, i64, i64, ci, ctypes.POINTER(QuantOut),
                                      ctypes.POINTER(QuantOut), vp]
    L.mxfp4_quantize_dual.restype = ci
    L.mxfp4_gemm.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, ctypes.c_float, vp, i64,
                             ci, vp, ctypes.c_size_t, vp]
    L.mxfp4_gemm.restype = ci
    L.mxfp4_gemm_ex.argtypes = [vp, i64, vp, i64, vp, i64, vp, i64, i64, i64, i64, ctypes.c_float, ctypes.c_float,
                                vp, ci, i64, ci, vp, ctypes.c_size_t, vp]
    L.mxfp4_gemm_ex.restype = ci
    L.mxfp4_quantize_dual_grouped.argtypes = [ctypes.POINTER(DualItem), ci, ci, vp]
    L.mxfp4_quantize_dual_grouped.restype = ci
    L.mxfp4_gemm_grouped.argtypes = [ctypes.POINTER(GemmItem), ci, i64, i64, i64, i64, i64, i64, i64,
                                     ctypes.c_float, i64, ci, vp]
    L.mxfp4_gemm_grouped.restype = ci
    L.mxfp4_gemm_workspace_bytes.argtypes = [i64, i64, i64]
    L.mxfp4_gemm_workspace_bytes.restype = ctypes.c_size_t
    L.mxfp4_tiled_sizes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.mxfp4_tiled_sizes.restype = ci
    L.mxfp4_linear_workspace_bytes.argtypes = [ci, i64, i64, i64]
    L.mxfp4_linear_workspace_bytes.restype = ctypes.c_size_t
    for name in ("mxfp4_linear_fprop", "mxfp4_linear_dgrad", "mxfp4_linear_wgrad"):
        f = getattr(L, name)
        f.argtypes = [vp, vp, i64, i64, i64, ctypes.POINTER(LinearCfg), vp, ctypes.c_size_t, vp, vp]
        f.restype = ci
    L.mxfp4_linear_step_workspace_bytes.argtypes = [i64, i64, i64]
    L.mxfp4_linear_step_workspace_bytes.restype = ctypes.c_size_t
    L.mxfp4_linear_forward.argtypes = [vp, vp, i64, i64, i64, ctypes.POINTER(StepCfg), vp, ctypes.c_size_t, vp, vp]
    L.mxfp4_linear_forward.restype = ci
    L.mxfp4_linear_backward.argtypes = [vp, i64, i64, i64, ctypes.POINTER(StepCfg), vp, ctypes.c_size_t, vp, vp,
                                        vp]
    L.mxfp4_linear_backward.restype = ci
    L.mxfp4_linear_fprop_noalloc.argtypes = [vp, vp, i64, i64, i64, ctypes.POINTER(LinearCfg), vp, vp]
    L.mxfp4_linear_fprop_noalloc.restype = ci
    L.mxfp4_status_string.argtypes = [ci]
    L.mxfp4_status_string.restype = ctypes.c_char_p
    L.mxfp4_abi_version.argtypes = []
    L.mxfp4_abi_version.restype = ci
    _lib = L
    return L


def _status_string(status):
    try:
        return lib().mxfp4_status_string(status).decode()
    except Exception:  # noqa: BLE001 - only used to format an error message
        return "status %d" % status


def _check(status, where):
    if status != 0:
        raise Mxfp4Error(status, where)


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _rounding(r):
    """'rne' / 'sr' (or RNE / SR), optionally '+noclip' (or | SCALE_NOCLIP) for the no-clip scale."""
    if isinstance(r, str):
        base, _, extra = r.partition("+")
        if extra not in ("", "noclip"):
            raise ValueError("rounding must be 'rne' or 'sr', optionally '+noclip'")
        flag = SCALE_NOCLIP if extra else 0
        if base in ("rne", "nearest"):
            return RNE | flag
        if base in ("sr", "stochastic"):
            return SR | flag
        raise ValueError("rounding must be 'rne' or 'sr', optionally '+noclip'")
    if int(r) & ~SCALE_NOCLIP in (RNE, SR):
        return int(r)
    raise ValueError("rounding must be RNE or SR, optionally | SCALE_NOCLIP")


def _layout(layout):
    if layout in (ROWS, "rows"):
        return ROWS
    if layout in (TILED, "tiled"):
        return TILED
    raise ValueError("layout must be 'rows' or 'tiled'")


def tiled_sizes(outer, L):
    """(codes bytes, scales bytes) of a tiled operand with `outer` rows of length L."""
    cb, sb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().mxfp4_tiled_sizes(int(outer), int(L), ctypes.byref(cb), ctypes.byref(sb)), "mxfp4_tiled_sizes")
    return cb.value, sb.value


def _require_cuda(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError("%s must be a tensor on a HIP device" % name)


def quantize(x, axis=1, hadamard=16, rounding="rne", seed=0, stream_id=0, q=None, scales=None,
             stream=None, layout="rows"):
    """Rotate then quantize a 2-D bf16/f32 device tensor to MXFP4.

    Returns (q, scales) uint8 tensors. Row layout: q [outer, L/2], scales [outer, L/32]; axis=0
    gives the quantized transpose (outer = columns). Tiled layout: the same bytes per row but rows
    padded to a multiple of 256 and arranged as include/mxfp4.h describes.
    """
    lay = _layout(layout)
    _require_cuda(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dtype = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dtype is None:
        raise TypeError("x must be bfloat16 or float32")
    rows, cols = x.shape
    L, outer = (cols, rows) if axis == 1 else (rows, cols)
    padded = (outer + 255) // 256 * 256 if lay == TILED else outer
    if q is None:
        q = torch.empty((padded, L // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((padded, L // 32), dtype=torch.uint8, device=x.device)
    st = lib().mxfp4_quantize(x.data_ptr(), dtype, rows, cols, x.stride(0), axis, hadamard,
                              _rounding(rounding), int(seed) & (2 ** 64 - 1), int(stream_id), lay,
                              q.data_ptr(), q.stride(0) if q.dim() == 2 else 0, scales.data_ptr(),
                              scales.stride(0) if scales.dim() == 2 else 0, _stream(stream))
    _check(st, "mxfp4_quantize")
    return q, scales


def _dual_out(x, spec, axis):
    """Output buffers and mxfp4_quant_out_t for one axis of quantize_dual."""
    spec = dict(spec or {})
    lay = _layout(spec.get("layout", "rows"))
    rows, cols = x.shape
    L, outer = (cols, rows) if axis == 1 else (rows, cols)
    padded = (outer + 255) // 256 * 256 if lay == TILED else outer
    q = spec.get("q")
    s = spec.get("scales")
    if q is None:
        q = torch.empty((padded, L // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((padded, L // 32), dtype=torch.uint8, device=x.device)
    out = QuantOut(_rounding(spec.get("rounding", "rne")), int(spec.get("seed", 0)) & (2 ** 64 - 1),
                   int(spec.get("stream_id", 0)), lay, q.data_ptr(), q.stride(0) if q.dim() == 2 else 0,
                   s.data_ptr(), s.stride(0) if s.dim() == 2 else 0)
    return q, s, out


def quantize_dual(x, hadamard=16, axis1=None, axis0=None, stream=None):
    """Both quantizations of x in one pass: along each row (axis1) and along each column (axis0,
    the quantized transpose). axis1 / axis0 are dicts with the optional keys rounding, seed,
    stream_id, layout, q, scales, meaning what quantize() takes. Returns (q1, s1, q0, s0),
    bit-identical to quantize(x, 1, ...) and quantize(x, 0, ...)."""
    _require_cuda(x, "x")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit column stride")
    dtype = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
    if dtype is None:
        raise TypeError("x must be bfloat16 or float32")
    q1, s1, o1 = _dual_out(x, axis1, 1)
    q0, s0, o0 = _dual_out(x, axis0, 0)
    rows, cols = x.shape
    st = lib().mxfp4_quantize_dual(x.data_ptr(), dtype, rows, cols, x.stride(0), hadamard,
                                   ctypes.byref(o1), ctypes.byref(o0), _stream(stream))
    _check(st, "mxfp4_quantize_dual")
    return q1, s1, q0, s0


DUAL_GROUP_MAX = 8


def quantize_dual_grouped(items, hadamard=16, stream=None):
    """quantize_dual of several tensors in one launch: items is a list of (x, axis1, axis0) with
    the meanings quantize_dual gives them (all x of one dtype, at most DUAL_GROUP_MAX). Returns
    [(q1, s1, q0, s0)] per item, bit-identical to quantize_dual of each."""
    items = list(items)
    if not 0 < len(items) <= DUAL_GROUP_MAX:
        raise ValueError("1 to %d tensors per grouped launch" % DUAL_GROUP_MAX)
    outs, arr = [], (DualItem * len(items))()
    for i, (x, axis1, axis0) in enumerate(items):
        _require_cuda(x, "x")
        if x.dim() != 2 or x.stride(1) != 1:
            raise ValueError("x must be 2-D with unit column stride")
        dtype = {torch.bfloat16: BF16, torch.float32: F32}.get(x.dtype)
        if dtype is None:
            raise TypeError("x must be bfloat16 or float32")
        q1, s1, o1 = _dual_out(x, axis1, 1)
        q0, s0, o0 = _dual_out(x, axis0, 0)
        arr[i] = DualItem(x.data_ptr(), dtype, x.shape[0], x.shape[1], x.stride(0), o1, o0)
        outs.append((q1, s1, q0, s0))
    st = lib().mxfp4_quantize_dual_grouped(arr, len(items), hadamard, _stream(stream))
    _check(st, "mxfp4_quantize_dual_grouped")
    return outs


def _check_gemm_operands(aq, as_, bq, bs, M, N, K, lay):
    """Raise ValueError unless the operand tensors hold what an M x N x K product reads: codes
    [rows][K/2] and scales [rows][K/32] with rows >= M (A) and >= N (B), rounded up to 256 for
    the tiled layout (whose buffers are flat or [rows][...])."""
    if M < 0 or N < 0:
        raise ValueError("negative output size")
    for t, nm in ((aq, "aq"), (as_, "as"), (bq, "bq"), (bs, "bs")):
        if t.dtype != torch.uint8:
            raise TypeError("%s must be uint8" % nm)
        if t.stride(-1) != 1:
            raise ValueError("%s must have unit column stride" % nm)
    if lay == TILED:
        pm, pn = (M + 255) // 256 * 256, (N + 255) // 256 * 256
        for t, nm, rows, width in ((aq, "aq", pm, K // 2), (bq, "bq", pn, K // 2), (as_, "as", pm, K // 32),
                                   (bs, "bs", pn, K // 32)):
            if t.numel() < rows * width:
                raise ValueError("%s holds %d bytes; the tiled %d x %d operand needs %d" % (nm, t.numel(), rows, K,
                                                                                            rows * width))
        return
    if aq.dim() != 2 or bq.dim() != 2 or as_.dim() != 2 or bs.dim() != 2:
        raise ValueError("row-major operands must be 2-D")
    if bq.shape[1] * 2 != K:
        raise ValueError("aq and bq disagree on K (%d vs %d)" % (K, bq.shape[1] * 2))
    if K % 32:
        raise ValueError("K = %d is not a multiple of 32" % K)
    if as_.shape[1] != K // 32 or bs.shape[1] != K // 32:
        raise ValueError("scales must have K/32 = %d columns" % (K // 32))
    if aq.shape[0] < M or as_.shape[0] < M:
        raise ValueError("A operand has fewer than M = %d rows" % M)
    if bq.shape[0] < N or bs.shape[0] < N:
        raise ValueError("B operand has fewer than N = %d rows" % N)


def gemm_workspace_bytes(M, N, K) -> int:
    return int(lib().mxfp4_gemm_workspace_bytes(int(M), int(N), int(K)))


def gemm(aq, as_, bq, bs, alpha=1.0, out=None, stream=None, layout="rows", m=None, n=None,
         workspace=None, beta=0.0, out_dtype=None):
    """c[m][n] = alpha * sum_k deq(A)[m][k] deq(B)[n][k] + beta * c[m][n] (FP32 or bf16 [M, N]).

    Tiled operands are padded to 256 rows, so M and N come from `out`, or `m` and `n`. A device
    workspace of gemm_workspace_bytes(M, N, K) bytes lets few-tile products split K; "auto"
    allocates it. beta != 0 reads `out` (mxfp4_gemm_ex); a bf16 `out` (or out_dtype) gets the
    result rounded to nearest even."""
    lay = _layout(layout)
    for t, nm in ((aq, "aq"), (as_, "as"), (bq, "bq"), (bs, "bs")):
        _require_cuda(t, nm)
    M, K = aq.shape[0], aq.shape[1] * 2
    N = bq.shape[0]
    if out is not None:
        M, N = out.shape
    M = M if m is None else int(m)
    N = N if n is None else int(n)
    _check_gemm_operands(aq, as_, bq, bs, M, N, K, lay)
    if out is None:
        if beta != 0.0:
            raise ValueError("beta != 0 needs an existing `out`")
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=aq.device)
    if out.dtype not in (torch.float32, torch.bfloat16) or out.stride(-1) != 1:
        raise TypeError("out must be float32 or bfloat16 with unit column stride")
    if isinstance(workspace, str) and workspace == "auto":
        need = gemm_workspace_bytes(M, N, K)
        workspace = torch.empty(need, dtype=torch.uint8, device=aq.device) if need else None
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_len = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if out.dtype == torch.float32 and beta == 0.0:
        st = lib().mxfp4_gemm(aq.data_ptr(), aq.stride(0), as_.data_ptr(), as_.stride(0), bq.data_ptr(),
                              bq.stride(0), bs.data_ptr(), bs.stride(0), M, N, K, float(alpha),
                              out.data_ptr(), out.stride(0), lay, ws_ptr, ws_len, _stream(stream))
        _check(st, "mxfp4_gemm")
    else:
        st = lib().mxfp4_gemm_ex(aq.data_ptr(), aq.stride(0), as_.data_ptr(), as_.stride(0), bq.data_ptr(),
                                 bq.stride(0), bs.data_ptr(), bs.stride(0), M, N, K, float(alpha),
                                 float(beta), out.data_ptr(), 1 if out.dtype == torch.bfloat16 else 0,
                                 out.stride(0), lay, ws_ptr, ws_len, _stream(stream))
        _check(st, "mxfp4_gemm_ex")
    return out


GEMM_GROUP_MAX = 8


def gemm_grouped(items, alpha=1.0, outs=None, stream=None, layout="rows", m=None, n=None):
    """outs[i] = alpha * A_i B_i^T for items[i] = (aq, as, bq, bs), all of one shape, in one
    launch (mxfp4_gemm_grouped); each output equals what gemm() writes for that item. M and N
    come from `outs`, or `m` and `n` (tiled operands are padded)."""
    lay = _layout(layout)
    items = list(items)
    if not 0 < len(items) <= GEMM_GROUP_MAX:
        raise ValueError("1 to %d products per grouped launch" % GEMM_GROUP_MAX)
    aq0, as0, bq0, bs0 = items[0]
    M, K = aq0.shape[0], aq0.shape[1] * 2
    N = bq0.shape[0]
    if outs is not None:
        if len(outs) != len(items):
            raise ValueError("one output per product")
        M, N = outs[0].shape
    M = M if m is None else int(m)
    N = N if n is None else int(n)
    for it in items:
        for t, t0, nm in zip(it, items[0], ("aq", "as", "bq", "bs")):
            _require_cuda(t, nm)
            if t.shape != t0.shape or t.stride() != t0.stride():
                raise ValueError("grouped products must share operand shapes and strides (%s)" % nm)
        _check_gemm_operands(*it, M, N, K, lay)
    if outs is None:
        outs = [torch.empty((M, N), dtype=torch.float32, device=aq0.device) for _ in items]
    for o in outs:
        if o.dtype != torch.float32 or o.shape != (M, N) or o.stride() != outs[0].stride() or o.stride(-1) != 1:
            raise TypeError("outputs must be float32 [M, N] with one row stride")
    arr = (GemmItem * len(items))(*[GemmItem(a.data_ptr(), s.data_ptr(), b.data_ptr(), t.data_ptr(), o.data_ptr())
                                    for (a, s, b, t), o in zip(items, outs)])
    st = lib().mxfp4_gemm_grouped(arr, len(items), aq0.stride(0), as0.stride(0), bq0.stride(0), bs0.stride(0),
                                  M, N, K, float(alpha), outs[0].stride(0), lay, _stream(stream))
    _check(st, "mxfp4_gemm_grouped")
    return outs


def workspace_bytes(pass_, M, K, N) -> int:
    return int(lib().mxfp4_linear_workspace_bytes(int(pass_), int(M), int(K), int(N)))


def _linear(fn_name, pass_, a, b, M, K, N, out_shape, hadamard, rnd_a, rnd_b, seed, out, workspace,
            stream):
    _require_cuda(a, "first operand")
    _require_cuda(b, "second operand")
    for t in (a, b):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError("linear operands must be contiguous bfloat16")
    if out is None:
        out = torch.empty(out_shape, dtype=torch.float32, device=a.device)
    need = workspace_bytes(pass_, M, K, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    cfg = LinearCfg(int(hadamard), _rounding(rnd_a), _rounding(rnd_b), int(seed) & (2 ** 64 - 1))
    st = getattr(lib(), fn_name)(a.data_ptr(), b.data_ptr(), M, K, N, ctypes.byref(cfg),
                                 workspace.data_ptr(), workspace.numel(), out.data_ptr(),
                                 _stream(stream))
    _check(st, fn_name)
    return out


def linear_fprop(x, w, hadamard=16, rnd_a="rne", rnd_b="rne", seed=0, out=None, workspace=None,
                 stream=None):
    """Y[M,N] = X[M,K] W[N,K]^T with both operands rotated and quantized along K."""
    M, K = x.shape
    N = w.shape[0]
    return _linear("mxfp4_linear_fprop", FPROP, x, w, M, K, N, (M, N), hadamard, rnd_a, rnd_b,
                   seed, out, workspace, stream)


def linear_dgrad(dy, w, hadamard=16, rnd_a="rne", rnd_b="rne", seed=0, out=None, workspace=None,
                 stream=None):
    """dX[M,K] = dY[M,N] W[N,K] with both operands rotated and quantized along N."""
    M, N = dy.shape
    K = w.shape[1]
    return _linear("mxfp4_linear_dgrad", DGRAD, dy, w, M, K, N, (M, K), hadamard, rnd_a, rnd_b,
                   seed, out, workspace, stream)


def linear_wgrad(dy, x, hadamard=16, rnd_a="rne", rnd_b="rne", seed=0, out=None, workspace=None,
                 stream=None):
    """dW[N,K] = dY[M,N]^T X[M,K] with both operands rotated and quantized along the tokens M."""
    M, N = dy.shape
    K = x.shape[1]
    return _linear("mxfp4_linear_wgrad", WGRAD, dy, x, M, K, N, (N, K), hadamard, rnd_a, rnd_b,
                   seed, out, workspace, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # MXFP4_NOALLOC_SCRATCH_BYTES


def linear_fprop_noalloc(x, w, hadamard=16, rnd_a="rne", rnd_b="rne", seed=0, out=None, stream=None):
    """linear_fprop through mxfp4_linear_fprop_noalloc: the library's own per-device scratch array
    instead of a workspace (products needing more than NOALLOC_SCRATCH_BYTES are refused). Calls
    whose work overlaps on one GPU share that array and race."""
    _require_cuda(x, "x")
    _require_cuda(w, "w")
    for t in (x, w):
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError("linear operands must be contiguous bfloat16")
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    cfg = LinearCfg(int(hadamard), _rounding(rnd_a), _rounding(rnd_b), int(seed) & (2 ** 64 - 1))
    st = lib().mxfp4_linear_fprop_noalloc(x.data_ptr(), w.data_ptr(), M, K, N, ctypes.byref(cfg), out.data_ptr(),
                                          _stream(stream))
    _check(st, "mxfp4_linear_fprop_noalloc")
    return out


def step_workspace_bytes(M, K, N) -> int:
    return int(lib().mxfp4_linear_step_workspace_bytes(int(M), int(K), int(N)))


def _step_cfg(hadamard, fprop, dgrad, wgrad, seed):
    return StepCfg(int(hadamard), _rounding(fprop), _rounding(dgrad), _rounding(wgrad), int(seed) & (2 ** 64 - 1))


def linear_forward(x, w, hadamard=16, fprop="rne", dgrad="rne", wgrad="sr", seed=0, workspace=None, out=None,
                   stream=None):
    """Forward half of a training step: Y[M,N] = X W^T, with X and W each quantized once along
    both axes; the axes the backward products need stay in `workspace`. Returns (Y, workspace);
    pass the same workspace, unchanged, to linear_backward of the same step."""
    for t, name in ((x, "x"), (w, "w")):
        _require_cuda(t, name)
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError("%s must be contiguous bfloat16" % name)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError("x and w disagree on K")
    if workspace is None:
        workspace = torch.empty(max(step_workspace_bytes(M, K, N), 1), dtype=torch.uint8, device=x.device)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    cfg = _step_cfg(hadamard, fprop, dgrad, wgrad, seed)
    st = lib().mxfp4_linear_forward(x.data_ptr(), w.data_ptr(), M, K, N, ctypes.byref(cfg), workspace.data_ptr(),
                                    workspace.numel(), out.data_ptr(), _stream(stream))
    _check(st, "mxfp4_linear_forward")
    return out, workspace


def linear_backward(dy, K, workspace, hadamard=16, fprop="rne", dgrad="rne", wgrad="sr", seed=0, dx=None,
                    dw=None, stream=None):
    """Backward half of a training step: dX[M,K] = dY W and dW[N,K] = dY^T X from dY[M,N] and the
    workspace of the step's linear_forward call (same configuration). Returns (dX, dW)."""
    _require_cuda(dy, "dy")
    if dy.dtype != torch.bfloat16 or not dy.is_contiguous():
        raise TypeError("dy must be contiguous bfloat16")
    M, N = dy.shape
    if dx is None:
        dx = torch.empty((M, int(K)), dtype=torch.float32, device=dy.device)
    if dw is None:
        dw = torch.empty((N, int(K)), dtype=torch.float32, device=dy.device)
    cfg = _step_cfg(hadamard, fprop, dgrad, wgrad, seed)
    st = lib().mxfp4_linear_backward(dy.data_ptr(), M, int(K), N, ctypes.byref(cfg), workspace.data_ptr(),
                                     workspace.numel(), dx.data_ptr(), dw.data_ptr(), _stream(stream))
    _check(st, "mxfp4_linear_backward")
    return dx, dw

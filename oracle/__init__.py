"""CPU oracle for the MXFP4 + block-Hadamard linear-layer GEMMs (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package. It shares no code with the HIP library: the arithmetic lives in
``mxfp4_oracle.c`` (binary32 Hadamard and encoding, binary64 GEMM) and, for tiny inputs, in the
exact rational implementation of :mod:`oracle.exact`.

The three GEMMs follow the gist.science summary of "MXFP4 LLM pretraining", section 방법론
(Methodology): forward Y = X W^T, activation gradient dX = dY W and weight gradient
dW = dY^T X, each operand rotated by the deterministic block Hadamard along the GEMM's
contraction axis and then quantized to MXFP4 (the deterministic H16 on the whole pipeline,
section "주요 기여 및 발견" §2). alpha = 1/h undoes H H^T = h I.

Arrays are numpy: bf16 inputs are passed as uint16 bit patterns, f32 as float32.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("MXFP4_ORACLE_LIB") or _build.build(force=False)
    lib = ctypes.CDLL(path)
    i64, u64, u32, vp, c_int = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    lib.oracle_quantize.argtypes = [vp, c_int, i64, i64, i64, c_int, c_int, c_int, u64, u32, vp, vp]
    lib.oracle_quantize.restype = c_int
    lib.oracle_dequantize.argtypes = [vp, vp, i64, i64, vp]
    lib.oracle_dequantize.restype = None
    lib.oracle_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, ctypes.c_double, vp, vp]
    lib.oracle_gemm.restype = None
    lib.oracle_gemm_sampled.argtypes = [vp, vp, vp, vp, i64, ctypes.c_double, vp, vp, i64, vp, vp]
    lib.oracle_gemm_sampled.restype = None
    lib.oracle_philox4x32_10.argtypes = [vp, vp, vp]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_fwht_binary32.argtypes = [vp, i64, c_int]
    lib.oracle_fwht_binary32.restype = None
    lib.oracle_rht_signs.argtypes = [u64, i64, vp]
    lib.oracle_rht_signs.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = c_int
    _lib = lib
    return lib


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


RNE = 0
SR = 1
RHT = 0x100  # added to hadamard (16 or 32): randomized Hadamard, signs keyed by the seed
ORTHO = 0x200  # added to hadamard (16 or 32): orthonormal rotation H_h / sqrt(h)
NOCLIP = 0x10  # added to rounding: the smallest scale that maps the block maximum to <= 6


def num_threads() -> int:
    return _load().oracle_num_threads()


def philox4x32_10(counter, key):
    """Philox4x32-10 block: counter (4 x uint32), key (2 x uint32) -> 4 x uint32."""
    c = np.ascontiguousarray(counter, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def fwht(v, h):
    """Unnormalised Walsh-Hadamard transform in binary32 of each aligned group of h values."""
    a = np.array(v, dtype=np.float32, copy=True).reshape(-1)
    _load().oracle_fwht_binary32(_ptr(a), a.size, int(h))
    return a.reshape(np.shape(v))


def rht_signs(seed, count):
    """The randomized-Hadamard diagonal d_0 .. d_{count-1} (+1 / -1) for key ``seed``."""
    out = np.zeros(int(count), dtype=np.int8)
    _load().oracle_rht_signs(int(seed) & (2 ** 64 - 1), int(count), _ptr(out))
    return out


def quantize(x, axis=1, hadamard=16, rounding=RNE, seed=0, stream=0):
    """MXFP4-quantize a 2-D array along ``axis`` after the block Hadamard rotation
    (``hadamard`` 16 or 32, plus ``RHT``: the randomized Hadamard with signs keyed by ``seed``,
    and / or plus ``ORTHO``: the orthonormal H_h / sqrt(h)).

    x: uint16 (bf16 bit patterns) or float32, shape (rows, cols).
    Returns (codes uint8 [outer, L/2], scales uint8 [outer, L/32]) with L the quantized length
    and outer the other dimension (axis=0 yields the quantized transpose).
    """
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        dtype = 0
    elif x.dtype == np.float32:
        dtype = 1
    else:
        raise TypeError("x must be uint16 (bf16 bits) or float32")
    rows, cols = x.shape
    L, outer = (cols, rows) if axis == 1 else (rows, cols)
    if L % 32:
        raise ValueError("quantized length must be a multiple of 32")
    q = np.zeros((outer, L // 2), dtype=np.uint8)
    s = np.zeros((outer, L // 32), dtype=np.uint8)
    rc = _load().oracle_quantize(_ptr(x), dtype, rows, cols, cols, axis, hadamard, rounding,
                                 int(seed) & (2 ** 64 - 1), int(stream), _ptr(q), _ptr(s))
    if rc:
        raise RuntimeError("oracle_quantize failed (%d)" % rc)
    return q, s


def dequantize(q, s):
    """Decode codes [outer, L/2] and scales [outer, L/32] to binary64 [outer, L]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.uint8)
    outer, L = q.shape[0], q.shape[1] * 2
    out = np.empty((outer, L), dtype=np.float64)
    _load().oracle_dequantize(_ptr(q), _ptr(s), outer, L, _ptr(out))
    return out


def gemm(aq, as_, bq, bs, alpha=1.0, with_abs=False):
    """C = alpha * deq(A) deq(B)^T in binary64 (A: [M, K], B: [N, K]).

    with_abs also returns sum_k |alpha * deqA[m,k] * deqB[n,k]|, the tolerance basis.
    """
    aq, as_, bq, bs = (np.ascontiguousarray(t, dtype=np.uint8) for t in (aq, as_, bq, bs))
    M, K = aq.shape[0], aq.shape[1] * 2
    N = bq.shape[0]
    if bq.shape[1] * 2 != K:
        raise ValueError("contraction lengths differ")
    c = np.empty((M, N), dtype=np.float64)
    cabs = np.empty((M, N), dtype=np.float64) if with_abs else None
    _load().oracle_gemm(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), M, N, K, float(alpha), _ptr(c),
                        _ptr(cabs) if with_abs else None)
    return (c, cabs) if with_abs else c


def gemm_sampled(aq, as_, bq, bs, ms, ns, alpha=1.0):
    """Values and tolerance bases for the outputs (ms[i], ns[i]) only."""
    aq, as_, bq, bs = (np.ascontiguousarray(t, dtype=np.uint8) for t in (aq, as_, bq, bs))
    K = aq.shape[1] * 2
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    c = np.empty(ms.size, dtype=np.float64)
    cabs = np.empty(ms.size, dtype=np.float64)
    _load().oracle_gemm_sampled(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), K, float(alpha),
                                _ptr(ms), _ptr(ns), ms.size, _ptr(c), _ptr(cabs))
    return c, cabs


def alpha_for(hadamard):
    """H_h H_h^T = h I (and (H D)(H D)^T = h I for a +-1 diagonal D), so a product of two
    rotated operands carries a factor h; the orthonormal rotation H_h / sqrt(h) carries none."""
    if int(hadamard) & ORTHO:
        return 1.0
    h = int(hadamard) & ~RHT
    return 1.0 / h if h else 1.0


# ------------------------------------------------------------------ the three linear GEMMs --

def linear_fprop(x, w, hadamard=16, rnd_a=RNE, rnd_b=RNE, seed=0, with_abs=False):
    """Y[M,N] = X[M,K] W[N,K]^T; both operands rotated and quantized along K."""
    xa = quantize(x, 1, hadamard, rnd_a, seed, 0)
    wb = quantize(w, 1, hadamard, rnd_b, seed, 1)
    return gemm(*xa, *wb, alpha=alpha_for(hadamard), with_abs=with_abs)


def linear_dgrad(dy, w, hadamard=16, rnd_a=RNE, rnd_b=RNE, seed=0, with_abs=False):
    """dX[M,K] = dY[M,N] W[N,K]; dY along N (rows), W along N (columns -> transpose)."""
    a = quantize(dy, 1, hadamard, rnd_a, seed, 0)
    b = quantize(w, 0, hadamard, rnd_b, seed, 1)
    return gemm(*a, *b, alpha=alpha_for(hadamard), with_abs=with_abs)


def linear_wgrad(dy, x, hadamard=16, rnd_a=RNE, rnd_b=RNE, seed=0, with_abs=False):
    """dW[N,K] = dY[M,N]^T X[M,K]; both along the token axis M (transposed quantize)."""
    a = quantize(dy, 0, hadamard, rnd_a, seed, 0)
    b = quantize(x, 0, hadamard, rnd_b, seed, 1)
    return gemm(*a, *b, alpha=alpha_for(hadamard), with_abs=with_abs)

"""Thin ctypes binding over ``libmxfp4_ceiling.so`` (C ABI in ``include/mxfp4_ceiling.h``): the
HBM streaming and scaled-FP4 matrix-core kernels that measure the board's practical ceilings.
Arguments are torch tensors on the current device; calls enqueue on the current stream."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmxfp4_ceiling.so")
_lib = None

MFMA_FLOPS_PER_ROUND = 8 * 8 * 2 * 32 * 32 * 64  # per workgroup: 8 wavefronts x 8 MFMAs


def library_path() -> str:
    return _LIB_PATH


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError("%s is missing: build it with `python -m mxfp4_block_scaled_h16_amd.build`" % _LIB_PATH)
    L = ctypes.CDLL(_LIB_PATH)
    vp, sz, u32, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
    L.mxfp4_ceiling_read.argtypes = [vp, sz, u32, vp, vp]
    L.mxfp4_ceiling_write.argtypes = [vp, sz, u32, vp]
    L.mxfp4_ceiling_copy.argtypes = [vp, vp, sz, vp]
    L.mxfp4_ceiling_mfma.argtypes = [ci, ci, u32, vp, vp]
    for f in (L.mxfp4_ceiling_read, L.mxfp4_ceiling_write, L.mxfp4_ceiling_copy, L.mxfp4_ceiling_mfma):
        f.restype = ci
    _lib = L
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status, where):
    if status != 0:
        raise RuntimeError("%s failed (status %d)" % (where, status))


def _nbytes(t, what):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s: a contiguous device tensor is required" % what)
    return t.numel() * t.element_size()


def read(src, never, sink):
    """Stream every byte of src once; sink (one int32) is written only if a lane's XOR equals never."""
    _nbytes(sink, "read sink")
    _check(lib().mxfp4_ceiling_read(src.data_ptr(), _nbytes(src, "read"), never,
                                    sink.data_ptr(), _stream()), "mxfp4_ceiling_read")


def write(dst, pattern):
    _check(lib().mxfp4_ceiling_write(dst.data_ptr(), _nbytes(dst, "write"), pattern, _stream()),
           "mxfp4_ceiling_write")


def copy(src, dst):
    nbytes = _nbytes(src, "copy")
    if _nbytes(dst, "copy") < nbytes:
        raise ValueError("copy: destination smaller than source")
    _check(lib().mxfp4_ceiling_copy(src.data_ptr(), dst.data_ptr(), nbytes, _stream()), "mxfp4_ceiling_copy")


def mfma(workgroups, iters, seed, sink):
    """sink: float32 tensor of at least workgroups * 512 elements."""
    if sink.dtype != torch.float32 or _nbytes(sink, "mfma") < workgroups * 512 * 4:
        raise ValueError("mfma: sink must hold workgroups * 512 float32")
    _check(lib().mxfp4_ceiling_mfma(workgroups, iters, seed, sink.data_ptr(), _stream()), "mxfp4_ceiling_mfma")

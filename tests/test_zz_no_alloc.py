"""The allocation-free Fprop entry point (mxfp4_linear_fprop_noalloc), called through the C ABI:
bitwise the output of mxfp4_linear_fprop with a caller workspace, on two calls in a row (the
second smaller, so it reuses the library's device array after a larger product), and a product
whose workspace exceeds the array is refused before anything runs."""
import ctypes

import numpy as np
import pytest

from synth import inputs
from tests.gpu_util import announce, bf16_dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _lib():
    import mxfp4_block_scaled_h16_amd as mx
    return mx, mx.lib()


def _noalloc(mx, L, x, w, cfg):
    import torch
    M, K = x.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.float32, device=x.device)
    st = L.mxfp4_linear_fprop_noalloc(x.data_ptr(), w.data_ptr(), M, K, N, ctypes.byref(cfg), y.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, "mxfp4_linear_fprop_noalloc: %s" % L.mxfp4_status_string(st).decode()
    return y


@pytest.mark.parametrize("h,rnd", [(16, "rne"), (32, "sr")])
def test_noalloc_fprop_matches_the_workspace_call_twice(h, rnd):
    import torch
    mx, L = _lib()
    r = mx._rounding(rnd)
    cfg = mx.LinearCfg(h, r, r, 0x5EED)
    # the first product is the QKV projection's Fprop over 8192 tokens (768 output tiles: one
    # workgroup per CU walks them; 31 MB of quantized operands in the array); the second uses the
    # tiled layout and a split K (few output tiles); the third is smaller, row-major (K not a
    # multiple of 512); each runs after the previous one in the same array
    for M, K, N, seed in ((8192, 4096, 6144, 3), (512, 4096, 768, 1), (160, 224, 96, 2)):
        x, w, _ = inputs.linear_inputs(M, K, N, seed=seed)
        xd, wd = bf16_dev(x), bf16_dev(w)
        announce("noalloc fprop", M, K, N, "h", h, rnd)
        got = _noalloc(mx, L, xd, wd, cfg)
        ref = mx.linear_fprop(xd, wd, h, rnd, rnd, 0x5EED)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32)), (M, K, N)


def test_noalloc_refuses_products_beyond_the_array():
    import torch
    mx, L = _lib()
    limit = mx.NOALLOC_SCRATCH_BYTES
    M, K, N = 8192, 14336, 4096          # the down projection's Fprop: about 94 MB of operands
    assert mx.workspace_bytes(mx.FPROP, M, K, N) > limit
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    y = torch.full((4,), 7.0, dtype=torch.float32, device="cuda")
    cfg = mx.LinearCfg(16, 0, 0, 0)
    st = L.mxfp4_linear_fprop_noalloc(x.data_ptr(), x.data_ptr(), M, K, N, ctypes.byref(cfg), y.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 5, "expected MXFP4_ERR_WORKSPACE, got %d" % st
    torch.cuda.synchronize()
    assert (y.cpu() == 7.0).all()

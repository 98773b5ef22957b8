"""The training-step entry points (mxfp4_linear_forward / mxfp4_linear_backward): X, W and dY
each quantized once along both axes. Their outputs must be bitwise those of the three separate
linear calls with the same roundings and key (same quantized operands, same GEMM path), and
within the GEMM tolerance of the oracle; empty dimensions give empty or zero outputs."""
import numpy as np
import pytest

import oracle
from synth import inputs
from tests.gpu_util import announce, assert_gemm_close, bf16_dev, host, require_gpu

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _step(M, K, N, h, rnd, seed, what):
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(M + 3 * K + 7 * N + h)
    x = inputs.bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    w = inputs.bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    dy = inputs.bf16_bits((rng.standard_t(3, (M, N)) * 1e-3).astype(np.float32))
    fp, dg, wg = rnd
    announce("linear step", what, M, K, N, "h", h, "rnd", rnd)
    dx_, dw_, dy_ = bf16_dev(x), bf16_dev(w), bf16_dev(dy)
    y, ws = mx.linear_forward(dx_, dw_, h, fp, dg, wg, seed)
    gx, gw = mx.linear_backward(dy_, K, ws, h, fp, dg, wg, seed)
    sy = mx.linear_fprop(dx_, dw_, h, fp, fp, seed)
    sx = mx.linear_dgrad(dy_, dw_, h, dg, dg, seed)
    sw = mx.linear_wgrad(dy_, dx_, h, wg, wg, seed)
    return (x, w, dy), [host(t) for t in (y, gx, gw)], [host(t) for t in (sy, sx, sw)]


@pytest.mark.parametrize("M,K,N", [(256, 512, 384), (512, 1024, 512), (96, 160, 224)])
@pytest.mark.parametrize("h", [16, 32])
def test_step_equals_separate_calls_and_oracle(M, K, N, h):
    """Tiled and row-major operand layouts (each contraction tiled when a multiple of 512),
    nearest rounding for Fprop and Dgrad, Philox SR for Wgrad."""
    rnd = ("rne", "rne", "sr")
    (x, w, dy), got, sep = _step(M, K, N, h, rnd, 0x5EED, "layouts")
    for g, s_, name in zip(got, sep, ("fprop", "dgrad", "wgrad")):
        assert g.shape == s_.shape
        assert np.array_equal(g.view(np.uint32), s_.view(np.uint32)), "%s differs from the separate call" % name
    refs = (oracle.linear_fprop(x, w, h, with_abs=True),
            oracle.linear_dgrad(dy, w, h, with_abs=True),
            oracle.linear_wgrad(dy, x, h, oracle.SR, oracle.SR, 0x5EED, with_abs=True))
    for g, (ref, basis), name in zip(got, refs, ("fprop", "dgrad", "wgrad")):
        assert_gemm_close(g, ref, basis, TOL, "step " + name)


def test_step_flags_and_roundings():
    """Randomized orthonormal rotation with SR everywhere and the no-clip scale on Dgrad."""
    import mxfp4_block_scaled_h16_amd as mx
    rnd = ("sr", "rne+noclip", "sr")
    h = 32 | mx.RHT | mx.ORTHO
    _, got, sep = _step(256, 512, 512, h, rnd, 99, "flags")
    for g, s_ in zip(got, sep):
        assert np.array_equal(g.view(np.uint32), s_.view(np.uint32))


def test_step_qkv_full_size_sampled():
    """The Llama-3.1-8B QKV projection step (M=8192, K=4096, N=6144): bitwise equal to the
    separate calls on every output."""
    (x, w, dy), got, sep = _step(8192, 4096, 6144, 16, ("rne", "rne", "sr"), 0x5EED, "qkv")
    for g, s_ in zip(got, sep):
        assert np.array_equal(g.view(np.uint32), s_.view(np.uint32))


def test_step_empty_dimensions():
    import mxfp4_block_scaled_h16_amd as mx
    import torch
    dev = "cuda"
    for M, K, N in ((0, 64, 32), (64, 0, 32), (64, 32, 0)):
        announce("linear step empty", M, K, N)
        x = torch.zeros((M, K), dtype=torch.bfloat16, device=dev)
        w = torch.zeros((N, K), dtype=torch.bfloat16, device=dev)
        dy = torch.zeros((M, N), dtype=torch.bfloat16, device=dev)
        y = torch.full((M, N), float("nan"), device=dev)
        y, ws = mx.linear_forward(x, w, 16, out=y)
        dx = torch.full((M, K), float("nan"), device=dev)
        dw = torch.full((N, K), float("nan"), device=dev)
        dx, dw = mx.linear_backward(dy, K, ws, 16, dx=dx, dw=dw)
        torch.cuda.synchronize()
        for t in (y, dx, dw):
            assert t.numel() == 0 or bool((t == 0).all())

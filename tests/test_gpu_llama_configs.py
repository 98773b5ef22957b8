"""Full-size parity of the Llama-3.1-8B-shaped workloads, checked on sampled outputs.

Each case runs the linear entry point the benchmark times, at the full shape, and compares a
random sample of outputs (plus the four corners) with the oracle, which quantizes the same
operands on the host and evaluates only the sampled dot products. Bar: |c - c_ref| <=
1e-5 * alpha * sum_k |a_k b_k| per output."""
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


def sample_pairs(rows, cols, count, seed):
    rng = np.random.default_rng(seed)
    ms = np.concatenate([rng.integers(0, rows, count), [0, rows - 1, 0, rows - 1]])
    ns = np.concatenate([rng.integers(0, cols, count), [0, 0, cols - 1, cols - 1]])
    return ms, ns


def check_sampled(got, qa, qb, h, what, count=2048, seed=1):
    """got: GPU output [rows_A, rows_B]; qa / qb: oracle quantizations along the contraction."""
    ms, ns = sample_pairs(got.shape[0], got.shape[1], count, seed)
    ref, basis = oracle.gemm_sampled(*qa, *qb, ms, ns, alpha=oracle.alpha_for(h))
    return assert_gemm_close(got[ms, ns], ref, basis, TOL, what)


def test_gate_up_fprop_and_dgrad():
    """Fused gate+up projection, M=8192, K=4096, N=28672: Fprop along K, Dgrad along N=28672
    (the longest contraction of the layer). H16, RNE."""
    import mxfp4_block_scaled_h16_amd as mx
    M, K, N = 8192, 4096, 28672
    x, w, dy = inputs.linear_inputs(M, K, N, seed=0)
    xd, wd, dyd = bf16_dev(x), bf16_dev(w), bf16_dev(dy)
    announce("gate+up fprop", M, K, N)
    y = host(mx.linear_fprop(xd, wd, 16))
    check_sampled(y, oracle.quantize(x, 1, 16), oracle.quantize(w, 1, 16), 16, "gate+up fprop")
    del y
    announce("gate+up dgrad", M, K, N)
    dx = host(mx.linear_dgrad(dyd, wd, 16))
    check_sampled(dx, oracle.quantize(dy, 1, 16), oracle.quantize(w, 0, 16), 16, "gate+up dgrad")


@pytest.mark.parametrize("h", [16, 32])
def test_down_wgrad_token_axis(h):
    """Down projection weight gradient dW[4096, 14336] = dY[8192, 4096]^T X[8192, 14336]: both
    operands quantized along the 8192 tokens (transposed), RNE, H16 and H32."""
    import mxfp4_block_scaled_h16_amd as mx
    dy, x = inputs.down_wgrad(seed=0)
    announce("down wgrad", h)
    dw = host(mx.linear_wgrad(bf16_dev(dy), bf16_dev(x), h))
    check_sampled(dw, oracle.quantize(dy, 0, h), oracle.quantize(x, 0, h), h, "down wgrad h%d" % h)


@pytest.mark.timeout(900)
def test_llama_layer_all_projections_with_sr_wgrad():
    """One decoder layer: q, k, v, o, gate, up, down at 8192 tokens, Fprop + Dgrad + Wgrad each,
    H16, nearest-even on Fprop/Dgrad operands and Philox stochastic rounding (seed 0) on both
    Wgrad operands."""
    import mxfp4_block_scaled_h16_amd as mx
    acts, per_proj = inputs.llama_layer_inputs(seed=0)
    worst = {}
    for name, (k, n) in inputs.LLAMA31_8B_PROJECTIONS.items():
        x = acts[inputs.LLAMA31_8B_INPUT_OF[name]]
        w, dy = per_proj[name]
        assert x.shape == (8192, k) and w.shape == (n, k) and dy.shape == (8192, n)
        xd, wd, dyd = bf16_dev(x), bf16_dev(w), bf16_dev(dy)
        announce("layer", name, "fprop")
        got = host(mx.linear_fprop(xd, wd, 16))
        worst[name + " fprop"] = check_sampled(got, oracle.quantize(x, 1, 16), oracle.quantize(w, 1, 16), 16,
                                               name + " fprop", count=512)
        announce("layer", name, "dgrad")
        got = host(mx.linear_dgrad(dyd, wd, 16))
        worst[name + " dgrad"] = check_sampled(got, oracle.quantize(dy, 1, 16), oracle.quantize(w, 0, 16), 16,
                                               name + " dgrad", count=512)
        announce("layer", name, "wgrad sr")
        got = host(mx.linear_wgrad(dyd, xd, 16, "sr", "sr", 0))
        worst[name + " wgrad"] = check_sampled(
            got, oracle.quantize(dy, 0, 16, oracle.SR, 0, 0), oracle.quantize(x, 0, 16, oracle.SR, 0, 1), 16,
            name + " wgrad", count=512)
        del got, xd, wd, dyd
    print("worst |err| / (alpha sum|ab|) per GEMM:", {k: "%.2e" % v for k, v in worst.items()})

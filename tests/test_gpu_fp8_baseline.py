"""The vendor FP8 GEMMs the benchmark reports as the pages' FP8 baseline compute the intended
products: for per-tensor FP8 E4M3 and for MXFP8 (E8M0 scale per 32), at a small shape and at
sampled rows of a Llama-3.1-8B layer shape, the hipBLASLt result (bf16) equals the binary64 product
of its own operands decoded on the CPU.

The bar is the vendor's output precision, measured rather than assumed: its block-scaled result
is often one bf16 unit in the last place away from the correctly rounded product (about half of
the outputs of a 256 x 256 x 512 MXFP8 product differ from it, the largest by one unit, so the
conversion is not round-to-nearest), and its per-tensor product lands up to about 1.5e-5 *
sum|a b| from the exact value where terms cancel. So each output must be within one bf16 unit
(2^-7 |ref|) plus 2^-12 * sum|a b|, and the whole product within 2^-8 in relative Frobenius norm.
Wrong operands, scales or a transposed scale layout miss both by orders of magnitude."""
import numpy as np
import pytest

from synth import inputs
from tests.gpu_util import announce, bf16_dev, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _decode(codes, scale, per_block):
    """float64 values of FP8 E4M3 codes times their scale (per tensor, or per 32 along rows)."""
    import torch
    v = codes.cpu().to(torch.float64).numpy()
    s = scale.cpu()
    if per_block:
        e = s.view(torch.uint8).numpy().astype(np.float64) - 127.0
        return v * np.repeat(np.exp2(e), 32, axis=1)
    return v * float(s)


@pytest.mark.parametrize("kind", ["fp8", "mxfp8"])
@pytest.mark.parametrize("M,K,N,rows", [(256, 512, 256, None), (8192, 4096, 1024, 64)])
def test_vendor_fp8_gemm_matches_decoded_product(kind, M, K, N, rows):
    import torch
    import bench
    x, w, _ = inputs.linear_inputs(M, K, N, seed=4)
    X, W = bf16_dev(x), bf16_dev(w)
    conv = bench.fp8_per_tensor if kind == "fp8" else bench.mxfp8
    a, b = conv(X), conv(W)
    announce("vendor", kind, M, K, N)
    c = bench.vendor_gemm(kind, a, b).float().cpu().numpy().astype(np.float64)
    idx = np.arange(M) if rows is None else np.linspace(0, M - 1, rows).round().astype(np.int64)
    per_block = kind == "mxfp8"
    A = _decode(a[0][torch.from_numpy(idx).cuda()], a[1][torch.from_numpy(idx).cuda()] if per_block else a[1],
                per_block)
    B = _decode(b[0], b[1], per_block)
    ref = A @ B.T
    basis = np.abs(A) @ np.abs(B).T
    err = np.abs(c[idx] - ref)
    bound = 2.0 ** -7 * np.abs(ref) + 2.0 ** -12 * basis
    assert np.linalg.norm(c[idx] - ref) <= 2.0 ** -8 * np.linalg.norm(ref), kind
    assert (err <= bound).all(), "%s: %d outputs off, worst %.3e vs %.3e" % (
        kind, int((err > bound).sum()), err.max(), bound[np.unravel_index(np.argmax(err - bound), err.shape)])

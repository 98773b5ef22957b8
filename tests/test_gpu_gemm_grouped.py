"""Grouped launches (mxfp4_gemm_grouped): products of one shape whose tiles share one grid.

Each output must equal, bit for bit, what mxfp4_gemm writes for the same operands with an
unsplit contraction: both add the block products of an output in K order into one FP32 chain, or
into the same fixed segments when K exceeds 5120, whatever tile size the launch uses. And each
output must be within 1e-5 * sum|a b| of the oracle's exact product."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import announce, assert_gemm_close, host, require_gpu, tile

pytestmark = pytest.mark.gpu

TOL = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _operand(rng, outer, K):
    codes = rng.integers(0, 16, size=(outer, K), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = rng.integers(112, 140, size=(outer, K // 32), dtype=np.uint8)
    return q, s


def _products(count, M, N, K, layout, seed, shared_a=True):
    """Host operands (row-major) and their device copies in `layout`; A shared by all products
    when shared_a (the key and value projections read one input)."""
    rng = np.random.default_rng(seed)
    host_ops, dev_ops = [], []
    a = _operand(rng, M, K)
    for _ in range(count):
        if not shared_a:
            a = _operand(rng, M, K)
        b = _operand(rng, N, K)
        host_ops.append((a, b))
        if layout == "tiled":
            ra, rb = -(-M // 256) * 256, -(-N // 256) * 256
            da = [_dev(t.reshape(ra, -1)) for t in tile(*a, M, K)]
            db = [_dev(t.reshape(rb, -1)) for t in tile(*b, N, K)]
        else:
            da, db = [_dev(a[0]), _dev(a[1])], [_dev(b[0]), _dev(b[1])]
        dev_ops.append((da[0], da[1], db[0], db[1]))
    return host_ops, dev_ops


def _check(count, M, N, K, layout, alpha, seed, sample=None):
    import mxfp4_block_scaled_h16_amd as mx
    host_ops, dev_ops = _products(count, M, N, K, layout, seed)
    announce("gemm grouped", count, M, N, K, layout)
    outs = [host(c) for c in mx.gemm_grouped(dev_ops, alpha, layout=layout, m=M, n=N)]
    for i, ((a, b), ops) in enumerate(zip(host_ops, dev_ops)):
        single = host(mx.gemm(*ops, alpha=alpha, layout=layout, m=M, n=N))
        assert np.array_equal(outs[i].view(np.uint32), single.view(np.uint32)), \
            "product %d of the group differs from its own launch" % i
        if sample is None:
            ref, basis = oracle.gemm(*a, *b, alpha=alpha, with_abs=True)
            assert_gemm_close(outs[i], ref, basis, TOL, "grouped %d %dx%dx%d" % (i, M, N, K))
        else:
            rng = np.random.default_rng(seed + i)
            ms = np.concatenate([rng.integers(0, M, sample), [0, M - 1]])
            ns = np.concatenate([rng.integers(0, N, sample), [N - 1, 0]])
            ref, basis = oracle.gemm_sampled(*a, *b, ms, ns, alpha=alpha)
            assert_gemm_close(outs[i][ms, ns], ref, basis, TOL, "grouped %d %dx%dx%d sampled" % (i, M, N, K))


@pytest.mark.parametrize("count,M,N,K,layout", [
    (3, 300, 200, 1024, "rows"),      # ragged tiles, one FP32 chain per output
    (2, 70, 50, 96, "rows"),          # K not a multiple of 512: one row-kernel launch per product
    (8, 256, 256, 512, "tiled"),      # the largest group
    (2, 1000, 520, 2048, "tiled"),
    (1, 513, 257, 1024, "tiled"),
])
def test_grouped_matches_single_and_oracle(count, M, N, K, layout):
    _check(count, M, N, K, layout, 0.0625, count * 1000 + M + N + K)


@pytest.mark.parametrize("M,N,K", [
    (8192, 1024, 4096),   # key / value Fprop of Llama-3.1-8B over 8192 tokens: 256 x 256 tiles
    (1024, 4096, 8192),   # key / value Wgrad: segmented chains, 128 x 128 tiles
    (4096, 2304, 8192),   # segmented chains on the 256 x 128 tile
])
def test_grouped_layer_shapes(M, N, K):
    _check(2, M, N, K, "tiled", 0.0625, M + N + K, sample=1024)


def test_grouped_long_contraction_worst_case():
    """Adversarial operands whose exact sum a single FP32 chain over K = 8192 loses: the grouped
    launch keeps the same fixed segments as the single one."""
    import mxfp4_block_scaled_h16_amd as mx
    from tests.test_accumulation import adversarial_operands
    M, N, K = 1024, 512, 8192
    (aq, as_), (bq, bs) = adversarial_operands(M, N, K)
    ops = (_dev(aq), _dev(as_), _dev(bq), _dev(bs))
    announce("gemm grouped adversarial", M, N, K)
    outs = [host(c) for c in mx.gemm_grouped([ops, ops])]
    ref, basis = oracle.gemm(aq[:1], as_[:1], bq[:1], bs[:1], with_abs=True)
    for c in outs:
        assert_gemm_close(c, np.broadcast_to(ref, c.shape), np.broadcast_to(basis, c.shape), TOL,
                          "grouped adversarial")


def test_grouped_empty_and_zero_contraction():
    import torch
    import mxfp4_block_scaled_h16_amd as mx
    _, ops = _products(2, 64, 32, 64, "rows", 3)
    announce("gemm grouped K = 0 / M = 0")
    z = [o[:, :0] for o in ops[0]]
    outs = [torch.full((64, 32), 7.0, device="cuda") for _ in range(2)]
    mx.gemm_grouped([z, z], outs=outs)
    assert all(float(host(o).max()) == 0.0 and float(host(o).min()) == 0.0 for o in outs)
    empty = [torch.empty((0, 32), device="cuda") for _ in range(2)]
    mx.gemm_grouped(ops, outs=empty)

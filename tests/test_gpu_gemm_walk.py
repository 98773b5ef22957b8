"""Products with more tiles than CUs, FP32 output and an even number of 512-wide groups per
contraction: one workgroup per CU walks the tiles, loading the next tile's first stages while it
finishes the current one. Contractions up to 5120 walk 256 x 256 tiles; longer ones, whose
accumulation chains restart in fixed segments, walk 256 x 128 tiles.

Each output must be within 1e-5 * sum|a b| of the oracle's exact product, and equal to what the
one-tile-per-workgroup kernel writes for the same operands (the beta path of mxfp4_gemm_ex on a
zeroed output runs that kernel; both add the block products in K order into one FP32 chain, and
adding beta * 0 changes no nonzero value). Shapes cover ragged tile edges, a last round that
leaves most CUs idle, two groups per contraction (the shortest walk), both operand layouts and
grouped launches."""
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


def _device(q, s, outer, K, layout):
    if layout == "tiled":
        rows = -(-outer // 256) * 256
        return [_dev(t.reshape(rows, -1)) for t in tile(q, s, outer, K)]
    return [_dev(q), _dev(s)]


def _sample(rng, M, N, count):
    ms = np.concatenate([rng.integers(0, M, count), [0, M - 1, M - 1, 0]])
    ns = np.concatenate([rng.integers(0, N, count), [0, N - 1, 0, N - 1]])
    return ms, ns


@pytest.mark.parametrize("M,N,K,layout,full", [
    (4400, 4000, 1024, "rows", True),      # 18 x 16 = 288 tiles: a second round of 32; ragged edges
    (4352, 3856, 2048, "tiled", True),     # 17 x 16 = 272 tiles
    (8192, 4096, 4096, "tiled", False),    # the q / o projection's Fprop over 8192 tokens: 2 rounds
    (8192, 14336, 4096, "tiled", False),   # the gate Fprop: 7 rounds
    (65792, 256, 1024, "tiled", False),    # 257 x 1 tiles: one workgroup takes two, no XCD spread
    (200, 76800, 2048, "rows", False),     # 1 x 300 tiles, 200 of 256 rows
    (8192, 4096, 1024, "rows", False),     # the k / v Dgrad shape: 2 groups per contraction
    (4400, 4000, 1536, "tiled", True),     # 3 groups: one workgroup per tile instead
    (4096, 4096, 8192, "tiled", False),    # segmented chains: the q projection's Wgrad, 512 tiles
    (2304, 3968, 6144, "rows", False),     # segmented chains, 9 x 31 tiles, ragged
    (8192, 4096, 14336, "tiled", False),   # the down projection's Fprop: 1024 tiles
])
def test_walk_matches_oracle_and_tile_kernel(M, N, K, layout, full):
    import torch
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    a, b = _operand(rng, M, K), _operand(rng, N, K)
    da, db = _device(*a, M, K, layout), _device(*b, N, K, layout)
    announce("gemm walk", M, N, K, layout)
    got = host(mx.gemm(*da, *db, alpha=0.0625, layout=layout, m=M, n=N))
    ref_tile = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    mx.gemm(*da, *db, alpha=0.0625, out=ref_tile, layout=layout, beta=1.0)
    assert np.array_equal(got, host(ref_tile)), "walk and one-tile-per-workgroup kernels differ"
    if full:
        ref, basis = oracle.gemm(*a, *b, alpha=0.0625, with_abs=True)
        assert_gemm_close(got, ref, basis, TOL, "walk %dx%dx%d" % (M, N, K))
    else:
        ms, ns = _sample(rng, M, N, 1024)
        ref, basis = oracle.gemm_sampled(*a, *b, ms, ns, alpha=0.0625)
        assert_gemm_close(got[ms, ns], ref, basis, TOL, "walk %dx%dx%d sampled" % (M, N, K))


@pytest.mark.parametrize("count,M,N,K,layout", [
    (3, 2048, 4096, 2048, "tiled"),    # 3 x 128 tiles walked together; each alone fits one round
    (2, 8192, 4096, 1024, "rows"),     # the k / v Dgrad pair of the decoder layer
    (2, 2048, 4096, 8192, "tiled"),    # segmented chains, 2 x 256 tiles of 256 x 128
])
def test_grouped_walk(count, M, N, K, layout):
    import mxfp4_block_scaled_h16_amd as mx
    rng = np.random.default_rng(count * 10 + K)
    a = _operand(rng, M, K)
    da = _device(*a, M, K, layout)
    hosts, ops = [], []
    for _ in range(count):
        b = _operand(rng, N, K)
        hosts.append(b)
        ops.append(tuple(da) + tuple(_device(*b, N, K, layout)))
    announce("gemm grouped walk", count, M, N, K, layout)
    outs = [host(c) for c in mx.gemm_grouped(ops, 0.0625, layout=layout, m=M, n=N)]
    for i, (b, op) in enumerate(zip(hosts, ops)):
        single = host(mx.gemm(*op, alpha=0.0625, layout=layout, m=M, n=N))
        assert np.array_equal(outs[i].view(np.uint32), single.view(np.uint32)), "product %d" % i
        ms, ns = _sample(rng, M, N, 512)
        ref, basis = oracle.gemm_sampled(*a, *b, ms, ns, alpha=0.0625)
        assert_gemm_close(outs[i][ms, ns], ref, basis, TOL, "grouped walk %d" % i)


def test_walk_repeated_launches_agree():
    """Back-to-back launches into one output: the same bits every time (the walk's reuse of its
    LDS ring across tiles leaves nothing behind that changes a later tile)."""
    import torch
    import mxfp4_block_scaled_h16_amd as mx
    M, N, K = 4400, 4000, 2048
    rng = np.random.default_rng(5)
    a, b = _operand(rng, M, K), _operand(rng, N, K)
    da, db = _device(*a, M, K, "tiled"), _device(*b, N, K, "tiled")
    announce("gemm walk repeated", M, N, K)
    c = torch.empty((M, N), dtype=torch.float32, device="cuda")
    first = None
    for _ in range(4):
        c.fill_(float("nan"))
        mx.gemm(*da, *db, alpha=0.0625, out=c, layout="tiled")
        now = host(c)
        if first is None:
            first = now
            assert not np.isnan(first).any()
        assert np.array_equal(now.view(np.uint32), first.view(np.uint32))


def test_walk_long_contraction_worst_case():
    """Adversarial operands whose exact sum a single FP32 chain over K = 8192 loses (every output
    the same): the walk's segmented chains keep every output within the bound."""
    import mxfp4_block_scaled_h16_amd as mx
    from tests.test_accumulation import adversarial_operands
    M, N, K = 2304, 4096, 8192                 # 9 x 32 tiles of 256 x 128
    (aq, as_), (bq, bs) = adversarial_operands(M, N, K)
    announce("gemm walk adversarial", M, N, K)
    c = host(mx.gemm(_dev(aq), _dev(as_), _dev(bq), _dev(bs)))
    ref, basis = oracle.gemm(aq[:1], as_[:1], bq[:1], bs[:1], with_abs=True)
    assert_gemm_close(c, np.broadcast_to(ref, c.shape), np.broadcast_to(basis, c.shape), TOL, "walk adversarial")

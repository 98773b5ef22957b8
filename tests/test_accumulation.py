"""The GEMM's FP32 accumulation: how the block-scaled MFMAs round, and the 1e-5 * sum|a b| bound
at long contractions.

How the hardware accumulates (GPU tests below): a scaled FP4 MFMA adds its block products (one
per 32 K values, each an exact integer times a power of two) to the FP32 accumulator one at a
time in K order, rounding to nearest even after each. An output accumulated in one chain over K
values therefore goes through up to K/32 roundings, and the recursive-summation bound
D * 2^-24 * sum|terms| exceeds 1e-5 once D > 167, i.e. beyond K = 5344.

The operands below reach that worst case: the first block product is 1 and every later one adds
31 * 2^-29, just under half a unit in the last place of 1, so a chain that never restarts stays
at exactly 1 and loses every later block. At K = 6144 (the QKV Dgrad's contraction), 8192 (every
weight gradient over 8192 tokens), 14336 (down Fprop, gate and up Dgrad) and 28672 (fused
gate+up Dgrad) that misses the bound by 1.1x to 5.3x unless the kernel keeps its chains short and
combines them in a fixed order. The reference values come from the oracle (exact block products
summed in binary64)."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import announce, assert_gemm_close, host, require_gpu

ONE = 0x2  # E2M1 code of +1.0


@pytest.fixture()
def gpu():
    require_gpu()


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _block(ones):
    """16 code bytes of one 32-element block holding `ones` leading codes of +1.0, then zeros."""
    codes = np.zeros(32, dtype=np.uint8)
    codes[:ones] = ONE
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def adversarial_operands(rows_a, rows_b, K):
    """A[rows_a][K], B[rows_b][K] with every output equal to 1 + (K/32 - 1) * 31 * 2^-29."""
    nb = K // 32
    qa = np.tile(_block(31), (nb, 1))
    qa[0] = _block(32)                     # block 0: 32 ones at 2^(127 + 122 - 254) = 2^-5 -> 1
    sa = np.full(nb, 113, dtype=np.uint8)  # later blocks: 31 ones at 2^(113 + 112 - 254) = 2^-29
    sb = np.full(nb, 112, dtype=np.uint8)
    sa[0], sb[0] = 127, 122
    qb = np.tile(_block(32), (nb, 1))
    A = np.tile(qa.reshape(1, -1), (rows_a, 1)), np.tile(sa, (rows_a, 1))
    B = np.tile(qb.reshape(1, -1), (rows_b, 1)), np.tile(sb, (rows_b, 1))
    return A, B


def test_adversarial_operands_reach_the_worst_case():
    """CPU check of the construction: the exact value, and that one FP32 chain with a rounding
    per block stays at 1, within the bound at K = 5120 and outside it from K = 6144 on."""
    for K, ok in ((5120, True), (6144, False), (8192, False), (28672, False)):
        (aq, as_), (bq, bs) = adversarial_operands(1, 1, K)
        ref, basis = oracle.gemm(aq, as_, bq, bs, with_abs=True)
        assert ref[0, 0] == 1.0 + (K // 32 - 1) * 31 * 2.0 ** -29
        chain = np.float32(1.0)
        for _ in range(K // 32 - 1):
            chain = np.float32(chain + np.float32(31 * 2.0 ** -29))
        assert chain == np.float32(1.0)
        assert (abs(float(chain) - ref[0, 0]) <= 1e-5 * basis[0, 0]) == ok


# (M, N, K) pick the launch: 4096 x 2304 has 144 output tiles of 256 x 256 (segmented chains on
# 256 x 128 tiles; K = 10240 and 10752 put the segment boundaries at different groups), 2048 x
# 2048 has 64 (128 x 128 tiles), 256 x 256 splits K over workgroups -- unless a split's chain
# would itself be too long (K = 131072)
CASES = [(4096, 2304, 6144), (4096, 2304, 8192), (4096, 2304, 10240), (4096, 2304, 10752),
         (4096, 2304, 14336), (4096, 2304, 28672),
         (2048, 2048, 8192), (2048, 2048, 28672),
         (256, 256, 8192), (256, 256, 28672), (256, 256, 131072)]


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K", CASES)
def test_long_contraction_worst_case(gpu, M, N, K):
    import mxfp4_block_scaled_h16_amd as mx
    (aq, as_), (bq, bs) = adversarial_operands(M, N, K)
    announce("long-K adversarial", M, N, K)
    c = host(mx.gemm(_dev(aq), _dev(as_), _dev(bq), _dev(bs), workspace="auto"))
    # every row of A and B is the same, so one oracle row gives every output
    ref, basis = oracle.gemm(aq[:1], as_[:1], bq[:1], bs[:1], with_abs=True)
    assert_gemm_close(c, np.broadcast_to(ref, c.shape), np.broadcast_to(basis, c.shape), 1e-5,
                      "adversarial %dx%dx%d" % (M, N, K))


@pytest.mark.gpu
@pytest.mark.parametrize("K", [8192 + 32, 28672 + 32])
def test_long_contraction_row_kernel(gpu, K):
    """K not a multiple of 512: the row-major kernel without the DMA pipeline."""
    import mxfp4_block_scaled_h16_amd as mx
    (aq, as_), (bq, bs) = adversarial_operands(96, 160, K)
    announce("long-K adversarial, row kernel", K)
    c = host(mx.gemm(_dev(aq), _dev(as_), _dev(bq), _dev(bs)))
    ref, basis = oracle.gemm(aq[:1], as_[:1], bq[:1], bs[:1], with_abs=True)
    assert_gemm_close(c, np.broadcast_to(ref, c.shape), np.broadcast_to(basis, c.shape), 1e-5,
                      "adversarial row kernel K=%d" % K)


def _single_value_gemm(K, blocks):
    """C (32 x 32, all equal) for A rows whose 32-blocks hold blocks[b] = (ones, exponent): `ones`
    codes of +1.0 scaled by 2^exponent (None: an all-zero block); B is all +1.0 at scale 1."""
    import mxfp4_block_scaled_h16_amd as mx
    nb = K // 32
    qa = np.zeros((nb, 16), dtype=np.uint8)
    sa = np.full(nb, 127, dtype=np.uint8)
    for b, spec in enumerate(blocks):
        if spec is not None:
            qa[b] = _block(spec[0])
            sa[b] = 127 + spec[1]
    qb = np.tile(_block(32), (nb, 1))
    sb = np.full(nb, 127, dtype=np.uint8)
    aq, as_ = np.tile(qa.reshape(1, -1), (32, 1)), np.tile(sa, (32, 1))
    bq, bs = np.tile(qb.reshape(1, -1), (32, 1)), np.tile(sb, (32, 1))
    c = host(mx.gemm(_dev(aq), _dev(as_), _dev(bq), _dev(bs)))
    got = np.unique(c.view(np.uint32))
    assert got.size == 1, "outputs differ across the tile"
    exact = oracle.gemm(aq[:1], as_[:1], bq[:1], bs[:1])[0, 0]
    return got.view(np.float32)[0], exact


ULP = 2.0 ** -23   # unit in the last place of 1
ONE_BLOCK = (32, -5)
# One step adds block products to the accumulator. A value 1 plus x units in the last place
# exercises the rounding: to nearest with ties to even, x = 0.25, 0.5, 0.75, 1.5, 2.5 give 0, 0,
# 1, 2, 2 units; truncation would give 0, 0, 0, 1, 2.
ULP_CASES = [(1, -25, 0.25), (1, -24, 0.5), (3, -25, 0.75), (3, -24, 1.5), (5, -24, 2.5)]


@pytest.mark.gpu
@pytest.mark.parametrize("K,small_block", [(64, 1), (128, 2), (512, 14), (512, 15)])
@pytest.mark.parametrize("ones,exp,x", ULP_CASES)
def test_accumulation_rounds_to_nearest_even(gpu, K, small_block, ones, exp, x):
    """1 followed by a block of x * 2^-23, in the same MFMA (block 1) or a later one, rounds to
    nearest, ties to even (K = 64, 128: the row kernel; 512: the pipelined kernel)."""
    blocks = [ONE_BLOCK] + [None] * (K // 32 - 1)
    blocks[small_block] = (ones, exp)
    announce("accumulation rounding K", K, "block", small_block, "x", x)
    got, exact = _single_value_gemm(K, blocks)
    assert exact == 1.0 + x * ULP
    assert got == np.float32(exact), "1 + %g ulp rounded to %r, nearest-even gives %r" % (x, got, np.float32(exact))


Q3 = (3, -26)   # 0.375 units in the last place of 1


@pytest.mark.gpu
@pytest.mark.parametrize("K,blocks,units", [
    # in one 64-wide MFMA step, after a previous step: the two blocks are not summed first
    (128, [ONE_BLOCK, None, Q3, Q3], 0),
    # inside the first step of the pipelined kernel, and across its two steps of a stage
    (512, [ONE_BLOCK, Q3, Q3, None] + [None] * 12, 0),
    (512, [ONE_BLOCK, None, Q3, Q3] + [None] * 12, 0),
    (512, [ONE_BLOCK, None, None, None, Q3, Q3, Q3, Q3] + [None] * 8, 0),
    # the same small blocks before the 1 add up exactly first and round it up
    (512, [Q3, Q3, ONE_BLOCK, None] + [None] * 12, 1),
])
def test_accumulation_rounds_after_every_block(gpu, K, blocks, units):
    """Each block product is added to the accumulator with its own rounding, in K order: blocks
    of 0.375 units in the last place after a 1 are each rounded away, while the same blocks
    before it first sum exactly to 0.75 units and then round 1 + 0.75 units up to 1 + 1 unit."""
    announce("per-block accumulation K", K, blocks)
    got, exact = _single_value_gemm(K, blocks)
    assert got == np.float32(1.0 + units * ULP), "got 1 + %g ulp (exact 1 + %g ulp)" % (
        (float(got) - 1.0) / ULP, (exact - 1.0) / ULP)

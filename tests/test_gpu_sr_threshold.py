"""Stochastic rounding at its decision boundary, through every quantizer kernel.

Each element's magnitude is built from its own random word r (Philox4x32-10 at its position in
the quantized output): the fractional position f between its grid neighbours has
floor(2^22 f) = floor(r / 2^10) (rounds down), the same with one more bit below the 22 kept
(still rounds down: the rule truncates f to 22 bits), or one 2^-22 unit more (rounds up). The
cases cycle through every binade of the E2M1 grid and both signs. Codes and scale bytes of the
row, column and dual kernels must equal the construction's and the oracle's bit for bit. Random
data almost never lands on these boundaries, so this pins the rounding rule itself.
"""
import numpy as np
import pytest

import oracle
from oracle import exact
from tests.gpu_util import announce, f32_dev, host, require_gpu

pytestmark = pytest.mark.gpu

SEED, STREAM = 0x5EED0F5EED, 1
ROWS, L = 256, 96


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _construct():
    """x [ROWS, L] float32 and the expected 4-bit codes along its rows (position i = o L + j)."""
    x = np.zeros((ROWS, L), dtype=np.float32)
    codes = np.zeros((ROWS, L), dtype=np.uint8)
    for o in range(ROWS):
        for j in range(L):
            neg = (7 * o + j) % 2 == 1
            if j % 32 == 0:
                a, mag = 4.0, 6           # block maximum: scale byte 127 (scale 1)
            else:
                r = exact.sr_word(SEED, STREAM, o * L + j)
                top = r >> 10
                case = (o + j) % 3
                f22 = top + 1 if case == 2 and top + 1 < 2 ** 22 else top
                t = 1 if case == 1 else 0  # a bit below the 22 the rule keeps
                region = j % 5
                if region == 0:            # [0, 0.5): lower neighbour 0, step 0.5
                    a, lo = (2 * f22 + t) * 2.0 ** -24, 0
                elif region == 1:          # [0.5, 1): lower neighbour 0.5, step 0.5
                    a, lo = 0.5 + (2 * f22 + t) * 2.0 ** -24, 1
                elif region == 2:          # [1, 2): step 0.5, f has exactly 22 bits
                    a, lo = 1.0 + f22 * 2.0 ** -23, 2
                elif region == 3:          # [2, 4): step 1
                    a, lo = 2.0 + f22 * 2.0 ** -22, 4
                else:                      # [4, 6): step 2
                    a, lo = 4.0 + f22 * 2.0 ** -21, 6
                mag = lo + (1 if f22 > top else 0)
            assert float(np.float32(a)) == a
            x[o, j] = -a if neg else a
            codes[o, j] = mag | (8 if neg else 0)
    return x, codes


def _unpack(q):
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


@pytest.fixture(scope="module")
def case():
    x, codes = _construct()
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=oracle.SR, seed=SEED, stream=STREAM)
    assert (s == 127).all()
    assert np.array_equal(_unpack(q), codes), "the oracle disagrees with the construction"
    return x, q, s


def _same(got_q, got_s, q, s, what):
    diff = got_q != q
    assert np.array_equal(got_s, s), "%s: scale bytes differ" % what
    assert not diff.any(), "%s: %d code bytes differ, first at %s" % (
        what, int(diff.sum()), np.argwhere(diff)[0])


def test_rows_kernel(case):
    import mxfp4_block_scaled_h16_amd as mx
    x, q, s = case
    announce("sr threshold rows", x.shape)
    gq, gs = mx.quantize(f32_dev(x), axis=1, hadamard=0, rounding="sr", seed=SEED, stream_id=STREAM)
    _same(host(gq), host(gs), q, s, "rows")


def test_cols_kernel(case):
    """Quantizing x^T along its first axis gives the same quantized rows (o, j) as x along its
    rows, with the same element positions and so the same random words."""
    import mxfp4_block_scaled_h16_amd as mx
    x, q, s = case
    xt = np.ascontiguousarray(x.T)
    announce("sr threshold cols", xt.shape)
    gq, gs = mx.quantize(f32_dev(xt), axis=0, hadamard=0, rounding="sr", seed=SEED, stream_id=STREAM)
    _same(host(gq), host(gs), q, s, "cols")


def test_dual_kernel(case):
    import mxfp4_block_scaled_h16_amd as mx
    x, q, s = case
    xt = np.ascontiguousarray(x.T)
    announce("sr threshold dual", xt.shape)
    q1, s1, q0, s0 = mx.quantize_dual(f32_dev(xt), 0, dict(rounding="sr", seed=SEED, stream_id=0),
                                      dict(rounding="sr", seed=SEED, stream_id=STREAM))
    _same(host(q0), host(s0), q, s, "dual, transposed output")
    rq, rs = oracle.quantize(xt, axis=1, hadamard=0, rounding=oracle.SR, seed=SEED, stream=0)
    _same(host(q1), host(s1), rq, rs, "dual, row output")


@pytest.mark.parametrize("d", [0, 1])
def test_published_zero_counter_block_in_every_kernel(d):
    """Seed 0, stream 0: the first four elements of quantized row 0 decide with the published
    Philox4x32-10 output words of counter 0 and key 0 (Salmon et al.), read from
    tests/golden/philox4x32_10_kat.txt, with no oracle involved: on their own word's threshold
    they round down, one 2^-22 unit above it they round up, in the row, column and dual kernels."""
    import mxfp4_block_scaled_h16_amd as mx
    from tests.test_oracle_pins import sr_kat_probe
    row, want = sr_kat_probe(d)
    x = np.zeros((32, 32), dtype=np.float32)
    x[:, 31] = 4.0
    x[0] = row[0]
    xt = np.ascontiguousarray(x.T)
    announce("sr published block, d =", d)
    gq, gs = mx.quantize(f32_dev(x), axis=1, hadamard=0, rounding="sr", seed=0, stream_id=0)
    cq, cs = mx.quantize(f32_dev(xt), axis=0, hadamard=0, rounding="sr", seed=0, stream_id=0)
    _, _, dq, ds = mx.quantize_dual(f32_dev(xt), 0, dict(rounding="rne"), dict(rounding="sr", seed=0, stream_id=0))
    for name, q, s in (("rows", gq, gs), ("cols", cq, cs), ("dual", dq, ds)):
        assert host(s)[0, 0] == 127, name
        assert list(_unpack(host(q))[0, :4]) == want, name

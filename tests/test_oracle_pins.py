"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test checks the oracle against something it does not compute itself: a library routine
(scipy's Hadamard, numpy's Philox, torch's E8M0 decode, the published Philox4x32-10
known answers), a closed form, a hand-derived table in
tests/golden/, exact rational brute force (oracle.exact), or an exact construction whose answer
is a plain matrix product. A plausible slip in the oracle (a dropped stage, a swapped sign or
index, a transposed operand, a wrong tie rule) fails at least one of them.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

import oracle
from oracle import exact
from synth import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def pack_codes(codes):
    """codes [outer, L] (0..15) -> packed bytes [outer, L/2], even element in the low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_codes(q):
    q = np.asarray(q, dtype=np.uint8)
    out = np.empty((q.shape[0], q.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = q & 15
    out[:, 1::2] = q >> 4
    return out


def e8m0_decode_torch(s):
    import torch
    t = torch.from_numpy(np.asarray(s, dtype=np.uint8).copy()).view(torch.float8_e8m0fnu)
    return t.to(torch.float64).numpy()


E2M1_FROM_GOLDEN = {int(c): float(v) for c, v in read_golden("e2m1_values.txt")}


def decode_independent(q, s):
    """Decode with the golden E2M1 table and torch's E8M0 conversion (not the oracle)."""
    codes = unpack_codes(q)
    vals = np.vectorize(lambda c: E2M1_FROM_GOLDEN[int(c)])(codes).astype(np.float64)
    sc = e8m0_decode_torch(s)
    return vals * np.repeat(sc, 32, axis=1)


# ----------------------------------------------------------------------------- format tables --

def test_e2m1_table_matches_golden_and_closed_form():
    # every code under the unit scale (byte 127)
    q = pack_codes(np.tile(np.arange(16, dtype=np.uint8), 2).reshape(1, 32))
    s = np.full((1, 1), 127, dtype=np.uint8)
    deq = oracle.dequantize(q, s)[0]
    for code in range(16):
        expect = E2M1_FROM_GOLDEN[code]
        assert deq[code] == expect
        assert math.copysign(1.0, deq[code]) == math.copysign(1.0, expect)
        # closed form: sign, exponent field (bias 1, subnormal at 0), mantissa bit
        sign, e, m = code >> 3, (code >> 1) & 3, code & 1
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2)
        assert abs(expect) == mag and (sign == 1) == (math.copysign(1.0, expect) < 0)


def test_e8m0_scale_decode_matches_torch():
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    q = pack_codes(np.full((256, 32), 2, dtype=np.uint8))  # code 2 = 1.0
    deq = oracle.dequantize(q, scales)
    ref = e8m0_decode_torch(scales)[:, 0]
    for s in range(255):
        assert deq[s, 0] == ref[s] == 2.0 ** (s - 127)
    assert np.isnan(deq[255, 0]) and np.isnan(ref[255])


# ----------------------------------------------------------------------------- Hadamard -------

@pytest.mark.parametrize("h", [16, 32])
def test_fwht_of_identity_is_scipy_hadamard(h):
    eye = np.eye(h, dtype=np.float32)
    rows = np.stack([oracle.fwht(eye[j], h) for j in range(h)])  # row j = H e_j = column j
    H = scipy.linalg.hadamard(h)
    assert np.array_equal(rows.T, H.astype(np.float32))
    assert np.array_equal(H @ H.T, h * np.eye(h, dtype=H.dtype))  # H^T H = h I


@pytest.mark.parametrize("h", [16, 32])
def test_fwht_exact_on_integers_and_involution(h):
    rng = np.random.default_rng(1)
    x = rng.integers(-1000, 1000, size=(64, h)).astype(np.float32)
    y = oracle.fwht(x, h)
    H = scipy.linalg.hadamard(h).astype(np.float64)
    assert np.array_equal(y.astype(np.float64), x.astype(np.float64) @ H.T)
    assert np.array_equal(oracle.fwht(y, h), h * x)
    # Parseval: |Hx|^2 = h |x|^2
    assert np.allclose((y.astype(np.float64) ** 2).sum(1), h * (x.astype(np.float64) ** 2).sum(1))


def test_fwht_binary32_rounding_order_matches_scalar_reference():
    """The fixed binary32 stage order (strides 1, 2, 4, ...; (u, w) -> (u + w, u - w)) checked
    with numpy float32 scalar arithmetic on values whose sums are inexact."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((200, 16)) * np.exp2(rng.integers(-30, 30, (200, 16)))).astype(np.float32)
    y = oracle.fwht(x, 16)
    for r in range(200):
        v = [np.float32(t) for t in x[r]]
        s = 1
        while s < 16:
            for i in range(16):
                if not i & s:
                    u, w = v[i], v[i + s]
                    v[i], v[i + s] = np.float32(u + w), np.float32(u - w)
            s *= 2
        assert np.array_equal(np.array(v, dtype=np.float32).view(np.uint32), y[r].view(np.uint32))


# ----------------------------------------------------------------------------- scale rule -----

def test_scale_rule_against_power_of_two_search():
    rng = np.random.default_rng(3)
    exps = rng.integers(-140, 128, size=400)
    amaxes = (rng.uniform(1, 2, size=400) * np.exp2(exps.astype(np.float64))).astype(np.float32)
    amaxes = amaxes[np.isfinite(amaxes) & (amaxes > 0)]
    extra = np.array([0, np.finfo(np.float32).max, np.finfo(np.float32).tiny, 1e-45, 4.0, 8.0,
                      7.999999, 3.9999998, 6.0, 2.0 ** -125, 2.0 ** -124], dtype=np.float32)
    amaxes = np.concatenate([amaxes, extra])
    x = np.zeros((amaxes.size, 32), dtype=np.float32)
    x[:, 5] = -amaxes
    x[:, 7] = amaxes / 3
    _, s = oracle.quantize(x, axis=1, hadamard=0)
    for a, got in zip(amaxes, s[:, 0]):
        assert got == exact.e8m0_scale(Fraction(float(a))), float(a)
        if a > 0 and 1 <= got <= 254:
            p = Fraction(2) ** (int(got) - 127)
            if got > 1:  # not clamped at the bottom of the E8M0 range
                assert 4 * p <= Fraction(float(a)) < 8 * p


# ----------------------------------------------------------------------------- RNE encode -----

def _encode_with_unit_scale(values, rounding=0, seed=0):
    """Quantize each value v in a block whose amax is pinned to 4 (scale byte 127, so the scaled
    value is v itself) and return the 4-bit codes of the values."""
    values = np.asarray(values, dtype=np.float32)
    n = values.size
    per = 31
    nblk = (n + per - 1) // per
    x = np.zeros((nblk, 32), dtype=np.float32)
    flat = np.zeros(nblk * per, dtype=np.float32)
    flat[:n] = values
    x[:, 1:] = flat.reshape(nblk, per)
    x[:, 0] = 4.0
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=rounding, seed=seed)
    assert (s == 127).all()
    return unpack_codes(q)[:, 1:].reshape(-1)[:n]


def test_rne_golden_points():
    rows = read_golden("e2m1_rne_points.txt")
    vals = [float(r[0]) for r in rows]
    codes = _encode_with_unit_scale(vals)
    for (v, c), got in zip(rows, codes):
        assert got == int(c), (v, c, got)


def test_rne_against_brute_force_dense():
    """Every bf16 value with |v| in [2^-4, 8) plus fp32 neighbours of all midpoints and grid points."""
    vals = []
    for e in range(-4, 3):
        for m in range(128):
            vals.append((1 + m / 128) * 2.0 ** e)
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1, 1.5, 2, 3, 4, 6, 7]
    for t in mids:
        b = exact.f32_bits(t)
        for d in range(-3, 4):
            vals.append(exact.f32_from_bits(b + d))
    vals += [0.0, 1e-45, 2.0 ** -126, 2.0 ** -127, 7.99999]
    vals = np.array(vals + [-v for v in vals], dtype=np.float32)
    vals = vals[np.abs(vals) < 8]
    codes = _encode_with_unit_scale(vals)
    for v, got in zip(vals, codes):
        mag = exact.round_e2m1_nearest_even(Fraction(float(v)))
        sign = 8 if math.copysign(1.0, float(v)) < 0 else 0
        assert got == (sign | mag), (float(v), got)


def test_rne_against_brute_force_random():
    rng = np.random.default_rng(4)
    vals = (rng.uniform(-8, 8, 20000)).astype(np.float32)
    codes = _encode_with_unit_scale(vals)
    for v, got in zip(vals, codes):
        mag = exact.round_e2m1_nearest_even(Fraction(float(v)))
        assert (got & 7) == mag and (got >> 3) == (1 if v < 0 or (v == 0 and math.copysign(1, v) < 0) else 0)


# ----------------------------------------------------------------------------- round trip -----

@pytest.mark.parametrize("h", [0, 16, 32])
def test_round_trip_error_bound(h):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-8, 8, (64, 1)))).astype(np.float32)
    q, s = oracle.quantize(x, axis=1, hadamard=h)
    deq = oracle.dequantize(q, s)
    y = oracle.fwht(x, h) if h else x
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    v = np.abs(y.astype(np.float64)) / scale
    half_spacing = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    bound = np.where(v > 6, v - 6, half_spacing) * scale
    assert (np.abs(y - deq) <= bound).all()


@pytest.mark.parametrize("rounding", [0, 1])
def test_idempotent_on_grid(rounding):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((32, 128)).astype(np.float32) * 3
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=rounding, seed=11)
    deq = oracle.dequantize(q, s).astype(np.float32)
    q2, s2 = oracle.quantize(deq, axis=1, hadamard=0, rounding=rounding, seed=99)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, q2)


# ----------------------------------------------------------------------------- conventions ----
# Conventions the pages leave open (parity unpinned by the pages; fixed by reading).

def test_nonfinite_zero_and_signed_zero_conventions():
    x = np.zeros((4, 32), dtype=np.float32)
    x[0, 3] = np.nan
    x[1, 9] = np.inf
    x[1, 10] = 1.0
    x[3, :] = -0.0
    x[3, 0] = 4.0
    x[3, 1] = -0.1
    q, s = oracle.quantize(x, axis=1, hadamard=0)
    assert s[0, 0] == 0xFF and s[1, 0] == 0xFF and (q[0] == 0).all() and (q[1] == 0).all()
    assert s[2, 0] == 0 and (q[2] == 0).all()
    codes = unpack_codes(q[3:4])[0]
    assert codes[0] == 6 and codes[1] == 8 and (codes[2:] == 8).all()


def test_axis0_is_axis1_of_transpose():
    rng = np.random.default_rng(7)
    t = inputs.bf16_bits(rng.standard_normal((96, 64)).astype(np.float32))
    for rounding in (0, 1):
        for h in (0, 16, 32):
            a = oracle.quantize(t, axis=0, hadamard=h, rounding=rounding, seed=5, stream=3)
            b = oracle.quantize(np.ascontiguousarray(t.T), axis=1, hadamard=h, rounding=rounding,
                                seed=5, stream=3)
            assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ----------------------------------------------------------------------------- Philox --------

def test_philox_structure_pinned_by_numpy():
    """The width-generic Philox equals numpy's Philox4x64-10 (numpy's first block uses
    counter + 1), which pins the round function, key schedule and output order."""
    for key in ([1, 2], [0xDEADBEEF12345678, 0x0123456789ABCDEF]):
        bg = np.random.Philox(key=np.array(key, dtype=np.uint64), counter=[0, 0, 0, 0])
        raw = [int(v) for v in bg.random_raw(12)]
        for blk in range(3):
            assert exact.philox([blk + 1, 0, 0, 0], key, width=64) == raw[4 * blk:4 * blk + 4]


def test_philox_weyl_constants_closed_form():
    for width in (32, 64):
        _, _, w0, w1 = exact.PHILOX_CONSTANTS[width]
        assert w0 == exact.weyl_constant(width, "phi")
        assert w1 == exact.weyl_constant(width, "sqrt3")


def test_philox4x32_10_known_answers():
    """The 32-bit generator the stochastic rounding and the randomized signs draw from
    reproduces the published Philox4x32-10 known-answer vectors (tests/golden)."""
    rows = read_golden("philox4x32_10_kat.txt")
    assert len(rows) == 3
    for row in rows:
        v = [int(t, 16) for t in row]
        ctr, key, want = v[0:4], v[4:6], v[6:10]
        assert [int(w) for w in oracle.philox4x32_10(ctr, key)] == want
        assert exact.philox(ctr, key, 32) == want


def test_philox4x32_oracle_matches_generic():
    rng = np.random.default_rng(8)
    for _ in range(200):
        ctr = [int(v) for v in rng.integers(0, 2 ** 32, 4, dtype=np.uint64)]
        key = [int(v) for v in rng.integers(0, 2 ** 32, 2, dtype=np.uint64)]
        assert [int(v) for v in oracle.philox4x32_10(ctr, key)] == exact.philox(ctr, key, 32)


def test_sr_against_brute_force():
    rng = np.random.default_rng(9)
    x = rng.uniform(-7.9, 7.9, size=(8, 32)).astype(np.float32)
    x[:, 0] = 4.0
    seed, stream = 0x1234567890ABCDEF, 1
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=1, seed=seed, stream=stream)
    assert (s == 127).all()
    codes = unpack_codes(q)
    for o in range(8):
        for j in range(32):
            r = exact.sr_word(seed, stream, o * 32 + j)
            mag = exact.round_e2m1_stochastic(Fraction(float(x[o, j])), r)
            assert codes[o, j] == ((8 if x[o, j] < 0 else 0) | mag)


def test_sr_threshold_22_bits():
    """The rounding decision compares the top 22 bits of the element's random word r with the
    fractional position f truncated to 22 bits. With r a multiple of 2^10 and |v| = (r + d) 2^-33
    (grid step 1/2 below 1/2, so f = (r + d) 2^-32 exactly): d = 0 (equality) rounds down, d = 512
    (below the next 22-bit unit of f, truncated away) rounds down, d = 1024 (one unit more) rounds
    up to 0.5."""
    seed, stream = 2024, 0
    nblk = 8000
    x = np.zeros((nblk, 32), dtype=np.float32)
    x[:, 0] = 4.0
    picked = []
    for o in range(nblk):
        for j in range(1, 32):
            r = exact.sr_word(seed, stream, o * 32 + j)
            if r & 0x3FF == 0 and 0 < r < 2 ** 32 - 1024:
                picked.append((o, j, r))
    assert len(picked) > 150
    offsets = (0, 512, 1024)
    for idx, (o, j, r) in enumerate(picked):
        d = offsets[idx % 3]
        x[o, j] = np.float32((r + d) * 2.0 ** -33)
        assert float(x[o, j]) == (r + d) * 2.0 ** -33
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=1, seed=seed, stream=stream)
    codes = unpack_codes(q)
    for idx, (o, j, r) in enumerate(picked):
        expect = exact.round_e2m1_stochastic(Fraction(float(x[o, j])), r)
        assert expect == (1 if idx % 3 == 2 else 0)
        assert codes[o, j] == expect


def sr_kat_probe(d):
    """One 32-element row for the stochastic-rounding pin by the published zero-counter block:
    elements 0..3 sit at the rounding threshold of the top 22 bits of the Philox4x32-10 output
    words 0..3 for counter 0 and key 0 (tests/golden/philox4x32_10_kat.txt, first row), plus d
    units of 2^-23; element 31 is 4.0 so that the block's scale is 2^0 and the grid step below
    0.5 is 0.5. Returns (x, the expected magnitude codes of elements 0..3)."""
    words = [int(w, 16) for w in read_golden("philox4x32_10_kat.txt")[0][6:10]]
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 31] = 4.0
    for j, w in enumerate(words):
        x[0, j] = np.float32(((w >> 10) + d) * 2.0 ** -23)
        assert float(x[0, j]) == ((w >> 10) + d) * 2.0 ** -23
    # |v| = (r22 + d) 2^-23 below 0.5: f = |v| / 0.5, floor(2^22 f) = r22 + d, rounds up iff
    # r22 < r22 + d
    return x, [1 if d >= 1 else 0] * 4


@pytest.mark.parametrize("d", [0, 1])
def test_sr_words_follow_published_zero_counter_block(d):
    """With seed 0 and stream 0, the first four elements of row 0 draw words 0, 1, 2, 3 of
    Philox4x32-10 at counter 0 and key 0, whose values are published (Salmon et al.): each
    element placed exactly on its own word's threshold rounds down, one 2^-22 unit above it rounds
    up. A swapped word, a per-element counter or a wrong key moves some element's threshold and
    fails one of the two cases."""
    x, want = sr_kat_probe(d)
    q, s = oracle.quantize(x, axis=1, hadamard=0, rounding=oracle.SR, seed=0, stream=0)
    assert s[0, 0] == 127
    assert list(unpack_codes(q)[0, :4]) == want


def test_sr_unbiased_and_noisier_than_rne():
    """Mean of SR over many seeds equals the value (5 sigma); MSE(SR) >= MSE(RNE)."""
    rng = np.random.default_rng(10)
    base = rng.uniform(-6, 6, 31).astype(np.float32)
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 4.0
    x[0, 1:] = base
    n = 3000
    xs = np.repeat(x, n, axis=0)
    acc = np.zeros(31)
    mse_sr = 0.0
    q, s = oracle.quantize(xs, axis=1, hadamard=0, rounding=1, seed=77)
    deq = oracle.dequantize(q, s)[:, 1:]
    acc = deq.mean(0)
    mse_sr = ((deq - base) ** 2).mean()
    qr, sr = oracle.quantize(x, axis=1, hadamard=0)
    mse_rne = ((oracle.dequantize(qr, sr)[0, 1:] - base) ** 2).mean()
    spacing = np.where(np.abs(base) < 2, 0.5, np.where(np.abs(base) < 4, 1.0, 2.0))
    sigma = spacing / 2 / math.sqrt(n)
    assert (np.abs(acc - base) <= 5 * sigma + 1e-12).all()
    assert mse_sr >= mse_rne


# ----------------------------------------------------------------------------- GEMM ----------

def _random_quantized(rng, outer, L):
    codes = rng.integers(0, 16, size=(outer, L), dtype=np.uint8)
    scales = rng.integers(110, 140, size=(outer, L // 32), dtype=np.uint8)
    return pack_codes(codes), scales


def test_gemm_unit_scales_is_integer_matmul():
    rng = np.random.default_rng(11)
    aq, _ = _random_quantized(rng, 7, 96)
    bq, _ = _random_quantized(rng, 5, 96)
    ones_a = np.full((7, 3), 127, dtype=np.uint8)
    ones_b = np.full((5, 3), 127, dtype=np.uint8)
    c = oracle.gemm(aq, ones_a, bq, ones_b)
    tv = np.vectorize(lambda k: int(round(2 * E2M1_FROM_GOLDEN[int(k)])))
    ia = tv(unpack_codes(aq)).astype(np.int64)
    ib = tv(unpack_codes(bq)).astype(np.int64)
    assert np.array_equal(c * 4, (ia @ ib.T).astype(np.float64))


def test_gemm_against_numpy_on_independent_decode():
    rng = np.random.default_rng(12)
    aq, as_ = _random_quantized(rng, 33, 160)
    bq, bs = _random_quantized(rng, 17, 160)
    c, cabs = oracle.gemm(aq, as_, bq, bs, alpha=1 / 16, with_abs=True)
    da = decode_independent(aq, as_)
    db = decode_independent(bq, bs)
    ref = (da @ db.T) / 16
    assert np.allclose(c, ref, rtol=1e-12, atol=0)
    assert np.allclose(cabs, np.abs(da) @ np.abs(db).T / 16, rtol=1e-12, atol=0)


def test_gemm_tiny_exact_rational():
    rng = np.random.default_rng(13)
    aq, as_ = _random_quantized(rng, 3, 64)
    bq, bs = _random_quantized(rng, 2, 64)
    c = oracle.gemm(aq, as_, bq, bs, alpha=1 / 32)
    ex = exact.gemm_exact(unpack_codes(aq).tolist(), as_.tolist(), unpack_codes(bq).tolist(),
                          bs.tolist(), Fraction(1, 32))
    for m in range(3):
        for n in range(2):
            assert c[m, n] == float(ex[m][n])


def test_gemm_nan_scale_propagates():
    rng = np.random.default_rng(14)
    aq, as_ = _random_quantized(rng, 4, 64)
    bq, bs = _random_quantized(rng, 3, 64)
    as_[2, 1] = 0xFF
    c = oracle.gemm(aq, as_, bq, bs)
    assert np.isnan(c[2]).all() and np.isfinite(np.delete(c, 2, axis=0)).all()


def test_gemm_sampled_matches_full():
    rng = np.random.default_rng(15)
    aq, as_ = _random_quantized(rng, 20, 128)
    bq, bs = _random_quantized(rng, 9, 128)
    c, cabs = oracle.gemm(aq, as_, bq, bs, alpha=0.5, with_abs=True)
    ms = rng.integers(0, 20, 30)
    ns = rng.integers(0, 9, 30)
    v, vabs = oracle.gemm_sampled(aq, as_, bq, bs, ms, ns, alpha=0.5)
    assert np.array_equal(v, c[ms, ns]) and np.array_equal(vabs, cabs[ms, ns])


# ----------------------------------------------------------------------------- end to end ----

def _exact_rotated_operand(rng, rows, K, h):
    """X = U H / h blockwise with U on the E2M1 grid (each 32-block max in {4, 6} times a block
    power of two), so rotating X recovers U exactly and MXFP4 represents it losslessly."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    U = grid[rng.integers(0, 8, size=(rows, K))] * rng.choice([-1, 1], size=(rows, K))
    U[:, ::32] = rng.choice([4.0, 6.0, -4.0, -6.0], size=(rows, K // 32))
    U *= np.repeat(np.exp2(rng.integers(-3, 4, size=(rows, K // 32))), 32, axis=1)
    H = scipy.linalg.hadamard(h).astype(np.float64)
    X = (U.reshape(rows, K // h, h) @ H.T / h).reshape(rows, K)
    return X, U


@pytest.mark.parametrize("h", [16, 32])
def test_end_to_end_exact_construction(h):
    """Linear forward on inputs where rotation + MXFP4 are lossless equals plain X W^T."""
    rng = np.random.default_rng(16)
    M, N, K = 24, 40, 128
    X, _ = _exact_rotated_operand(rng, M, K, h)
    W, _ = _exact_rotated_operand(rng, N, K, h)
    if h == 16:
        xb, wb = inputs.bf16_bits(X.astype(np.float32)), inputs.bf16_bits(W.astype(np.float32))
        assert np.array_equal(inputs.bf16_to_f32(xb), X.astype(np.float32))  # bf16-exact
        y = oracle.linear_fprop(xb, wb, hadamard=h)
    else:
        y = oracle.linear_fprop(X.astype(np.float32), W.astype(np.float32), hadamard=h)
    assert np.allclose(y, X @ W.T, rtol=1e-12, atol=1e-12)


def test_dgrad_wgrad_operand_orientation():
    """dX = dY W and dW = dY^T X, with exact operands (h = 0, values on the grid)."""
    rng = np.random.default_rng(17)
    M, N, K = 64, 96, 32
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    def exact_mat(r, c):
        a = grid[rng.integers(0, 8, (r, c))] * rng.choice([-1, 1], (r, c)).astype(np.float32)
        a[::32, :] = 6.0
        a[:, ::32] = 6.0
        return a
    dy, w, x = exact_mat(M, N), exact_mat(N, K), exact_mat(M, K)
    assert np.array_equal(oracle.linear_dgrad(dy, w, hadamard=0), dy.astype(np.float64) @ w)
    assert np.array_equal(oracle.linear_wgrad(dy, x, hadamard=0), dy.T.astype(np.float64) @ x)
    assert np.array_equal(oracle.linear_fprop(x, w, hadamard=0), x.astype(np.float64) @ w.T)


def test_rotation_lowers_error_on_outlier_activations():
    """Diagnostic in the direction of the method's finding (deterministic rotation corrects the
    structural micro-scaling error): relative error of the forward GEMM with H16 < without."""
    x, w = inputs.small_fprop(0)
    rng = np.random.default_rng(18)
    xf = inputs.bf16_to_f32(x).copy()
    xf[:, rng.choice(512, 2, replace=False)] *= 50
    xb = inputs.bf16_bits(xf)
    ref = inputs.bf16_to_f32(xb).astype(np.float64) @ inputs.bf16_to_f32(w).astype(np.float64).T
    err = {h: np.linalg.norm(oracle.linear_fprop(xb, w, hadamard=h) - ref) / np.linalg.norm(ref)
           for h in (0, 16)}
    assert err[16] < err[0]


# ----------------------------------------------------------------- randomized Hadamard ------

@pytest.mark.parametrize("h", [16, 32])
def test_rht_exact_construction(h):
    """X = d .* (U H / h) blockwise, with d the oracle's own sign diagonal: the randomized
    rotation must recover U exactly (lossless MXFP4) and the forward GEMM of two such operands
    (same key) must equal the plain product X W^T. Applying d after H, indexing it by the outer
    dimension, or giving the two operands different signs all break this."""
    rng = np.random.default_rng(61)
    M, N, K = 24, 40, 256
    seed = 0xABCDEF12345
    d = oracle.rht_signs(seed, K).astype(np.float64)
    X, _ = _exact_rotated_operand(rng, M, K, h)
    W, _ = _exact_rotated_operand(rng, N, K, h)
    X, W = X * d, W * d
    y = oracle.linear_fprop(X.astype(np.float32), W.astype(np.float32), hadamard=h | oracle.RHT, seed=seed)
    assert np.allclose(y, X @ W.T, rtol=1e-12, atol=1e-12)
    # a different key gives different signs, and the construction no longer holds exactly
    y2 = oracle.linear_fprop(X.astype(np.float32), W.astype(np.float32), hadamard=h | oracle.RHT, seed=seed + 1)
    assert not np.allclose(y2, X @ W.T, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rounding", [0, 1])
def test_rht_is_h_of_sign_flipped_input(axis, rounding):
    """Randomized rotation = deterministic rotation of the input with its sign bits flipped where
    d_j = -1, j the position along the quantized axis (bf16 sign flips are exact)."""
    rng = np.random.default_rng(62)
    x = inputs.bf16_bits(rng.standard_normal((96, 160)).astype(np.float32))
    x = x[:, :128] if axis == 1 else x[:96, :]
    L = x.shape[1] if axis == 1 else x.shape[0]
    seed = 77
    d = oracle.rht_signs(seed, L)
    flip = np.where(d < 0, 0x8000, 0).astype(np.uint16)
    xf = x ^ (flip[None, :] if axis == 1 else flip[:, None])
    for h in (16, 32):
        a = oracle.quantize(x, axis, h | oracle.RHT, rounding, seed, 1)
        b = oracle.quantize(xf, axis, h, rounding, seed, 1)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_rht_signs_balanced_and_keyed():
    """The sign diagonal is a fair, key-dependent +-1 sequence: the count of -1 over 2^16
    positions is within 5 standard deviations of half, two keys disagree on about half the
    positions, and the same key reproduces the same signs."""
    n = 1 << 16
    a = oracle.rht_signs(1, n)
    b = oracle.rht_signs(2, n)
    assert set(np.unique(a)) <= {-1, 1}
    sd = math.sqrt(n) / 2
    assert abs(int((a < 0).sum()) - n / 2) < 5 * sd
    assert abs(int((a != b).sum()) - n / 2) < 5 * sd
    assert np.array_equal(a, oracle.rht_signs(1, n))
    # prefixes agree: the sign of position j does not depend on how many are requested
    assert np.array_equal(oracle.rht_signs(1, 200), a[:200])


# ----------------------------------------------------------------------- no-clip scale ------

def _noclip_scale_by_search(amax):
    """Smallest S in [0, 254] with amax <= 6 * 2^(S - 127), by exhaustive search (exact)."""
    if amax == 0.0:
        return 0
    for S in range(0, 255):
        if Fraction(amax) <= 6 * Fraction(2) ** (S - 127):
            return S
    return 254


def test_noclip_scale_is_the_smallest_without_saturation():
    """rounding | NOCLIP: every block's scale byte is the smallest with amax <= 6 * scale (found
    by search over all 255 values), and it differs from the default rule by 0 or 1."""
    rng = np.random.default_rng(91)
    blocks = []
    for m in (1.0, 1.25, 1.5, 1.5000001, 1.75, 1.9999999):     # block max mantissas around 1.5
        for e in (-130, -126, -125, -124, -3, 0, 5, 100, 126):
            b = (rng.standard_normal(32) * 0.4 * m * 2.0 ** e).astype(np.float32)
            b[rng.integers(0, 32)] = np.float32(m * 2.0 ** e) * (1 if rng.random() < 0.5 else -1)
            blocks.append(b)
    x = np.concatenate(blocks).reshape(len(blocks), 32).astype(np.float32)
    _, s_def = oracle.quantize(x, 1, 0, oracle.RNE)
    q_nc, s_nc = oracle.quantize(x, 1, 0, oracle.RNE | oracle.NOCLIP)
    for i in range(x.shape[0]):
        amax = float(np.max(np.abs(x[i].astype(np.float64))))
        assert s_nc[i, 0] == _noclip_scale_by_search(amax), (i, amax)
        assert int(s_nc[i, 0]) - int(s_def[i, 0]) in (0, 1)
    # nothing saturates: every decoded value is within half a grid step of the input
    deq = oracle.dequantize(q_nc, s_nc)
    sc = np.exp2(s_nc.astype(np.float64) - 127)
    assert np.all(np.abs(deq - x) <= np.repeat(sc, 32, axis=1) * 1.0 + 1e-300)


@pytest.mark.parametrize("rounding", [0, 1])
def test_noclip_equals_default_when_nothing_would_clip(rounding):
    """Blocks whose maximum maps to at most 6 under the default rule get identical bytes."""
    rng = np.random.default_rng(92)
    top = (1.5 * np.exp2(rng.integers(-4, 4, (64, 4)))).astype(np.float32)   # block max mantissa 1.5
    bound = np.repeat(top, 32, axis=1)
    x = np.clip(rng.standard_normal((64, 128)).astype(np.float32), -0.99 * bound, 0.99 * bound)
    x[:, ::32] = top                                                     # maps to exactly 6
    a = oracle.quantize(x, 1, 0, rounding, 3)
    b = oracle.quantize(x, 1, 0, rounding | oracle.NOCLIP, 3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------------ orthonormal rotation -----

@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rounding", [0, 1])
def test_ortho_h16_is_the_unnormalised_rotation_two_binades_down(axis, rounding):
    """H16 / 4 scales every rotated value by an exact power of two: the codes are those of the
    unnormalised H16 and every scale byte is 2 lower (normal-range inputs, so nothing underflows;
    the SR words are the same because they depend only on the position)."""
    rng = np.random.default_rng(93)
    x = inputs.bf16_bits((rng.standard_normal((64, 96)) * 3).astype(np.float32))
    a = oracle.quantize(x, axis, 16, rounding, 5, 1)
    b = oracle.quantize(x, axis, 16 | oracle.ORTHO, rounding, 5, 1)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].astype(int) - 2, b[1].astype(int))


@pytest.mark.parametrize("h", [16, 32])
def test_ortho_unit_vectors_closed_form(h):
    """x = e_k inside each h-group: H_h e_k / sqrt(h) is column k of H_h times 1/sqrt(h), so a
    block's amax is 1/sqrt(h), the scale byte 127 + floor(log2(1/sqrt(h))) - 2 (122 for h = 32,
    123 for h = 16), every magnitude 2^(127 - S) / sqrt(h) (5.66 -> 6 for h = 32, exactly 4 for
    h = 16) and the signs those of (-1)^popcount(j & k). Scaling by 1/h or not at all gives other
    bytes."""
    L = 64
    x = np.zeros((h, L), dtype=np.float32)
    for k in range(h):
        x[k, k::h] = 1.0      # e_k in every h-group of row k
    q, s = oracle.quantize(x, 1, h | oracle.ORTHO, 0)
    S = 127 + math.floor(math.log2(1.0 / math.sqrt(h))) - 2
    assert (s == S).all()
    mag = 2.0 ** (127 - S) / math.sqrt(h)
    want_mag = {16: 6, 32: 7}[h]            # 4.0 is index 6; 5.66 rounds to 6.0, index 7
    assert abs(mag - {16: 4.0, 32: 5.656854249492381}[h]) < 1e-12
    codes = unpack_codes(q)
    for k in range(h):
        for j in range(L):
            neg = bin((j % h) & k).count("1") % 2 == 1
            assert codes[k, j] == (8 if neg else 0) | want_mag


@pytest.mark.parametrize("h", [16, 32])
def test_ortho_keeps_the_norm_and_the_product(h):
    """An orthonormal rotation keeps each row's energy: the dequantized rows carry the input's
    sum of squares up to the MXFP4 error; and the forward GEMM of two orthonormally rotated
    operands needs no 1/h factor (alpha 1) to approximate X W^T."""
    rng = np.random.default_rng(94)
    x = rng.standard_normal((32, 256)).astype(np.float32)
    w = (rng.standard_normal((48, 256)) * 0.02).astype(np.float32)
    q, s = oracle.quantize(x, 1, h | oracle.ORTHO, 0)
    ratio = (oracle.dequantize(q, s) ** 2).sum(axis=1) / (x.astype(np.float64) ** 2).sum(axis=1)
    assert np.all(np.abs(ratio - 1.0) < 0.15), ratio
    assert oracle.alpha_for(h | oracle.ORTHO) == 1.0 and oracle.alpha_for(h | oracle.ORTHO | oracle.RHT) == 1.0
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    err = lambda y: np.linalg.norm(y - ref) / np.linalg.norm(ref)  # noqa: E731
    e_ortho = err(oracle.linear_fprop(x, w, h | oracle.ORTHO))
    e_plain = err(oracle.linear_fprop(x, w, h))
    # MXFP4 on both operands of a K = 256 product of Gaussians: ~17% relative error either way;
    # a product off by a factor h (a missing or doubled 1/h) would be off by 94% or more
    assert e_ortho < 0.3 and abs(e_ortho - e_plain) < 0.1, (e_ortho, e_plain)

"""Exact, brute-force definitions for tiny inputs (test infrastructure only).

Pure Python with ``fractions.Fraction``. Each function states a definition in its plainest
form, written independently of ``mxfp4_oracle.c``, so the two can check each other:

* E2M1 rounding as an argmin over the eight grid magnitudes with the tie going to the even code
  (OCP Microscaling Formats v1.0: conversion to E2M1 uses round-to-nearest-even and saturates).
* The E8M0 scale as a search over powers of two (OCP MX v1.0: the shared exponent is
  floor(log2 amax) minus the element format's largest exponent, 2 for E2M1).
* The GEMM as exact rational sums.
* Philox as one routine generic in the word width (Salmon et al., SC'11): the 64-bit instance
  equals numpy's Philox4x64-10, which pins the round structure the 32-bit instance shares.
"""
from fractions import Fraction
import math
import struct

E2M1_GRID = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def round_e2m1_nearest_even(v: Fraction) -> int:
    """Magnitude index of the grid value nearest to |v|; equal distances go to the even index."""
    a = abs(v)
    best = None
    for idx, g in enumerate(E2M1_GRID):
        d = abs(a - g)
        if best is None or d < best[0] or (d == best[0] and idx % 2 == 0):
            best = (d, idx)
    return best[1]


def round_e2m1_stochastic(v: Fraction, r: int) -> int:
    """Magnitude index after stochastic rounding with the 32-bit word r.

    |v| >= 6 saturates; otherwise |v| lies in [lo, hi) between two neighbouring grid values and
    rounds to hi exactly when floor(r / 2^10) < floor(2^22 (|v| - lo) / (hi - lo)).
    """
    a = abs(v)
    if a >= 6:
        return 7
    for idx in range(7):
        lo, hi = E2M1_GRID[idx], E2M1_GRID[idx + 1]
        if lo <= a < hi:
            f = (a - lo) / (hi - lo)
            return idx + 1 if (r >> 10) < math.floor(f * 2 ** 22) else idx
    raise AssertionError("unreachable")


def e8m0_scale(amax: Fraction, nonfinite: bool = False) -> int:
    """Scale byte S with 2^(S-127) the largest power of two p such that 4 p <= amax
    (clamped to [2^-127, 2^127]); 0xFF for a non-finite block, 0 for an all-zero block."""
    if nonfinite:
        return 0xFF
    if amax == 0:
        return 0
    e = -127
    while e < 127 and 4 * Fraction(2) ** (e + 1) <= amax:
        e += 1
    return e + 127


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(b: int) -> float:
    return struct.unpack("<f", struct.pack("<I", b & 0xFFFFFFFF))[0]


def bf16_to_float(b: int) -> float:
    return f32_from_bits((b & 0xFFFF) << 16)


def sylvester(h: int):
    """Sylvester Hadamard matrix with entries (-1)^popcount(i & j)."""
    return [[-1 if bin(i & j).count("1") % 2 else 1 for j in range(h)] for i in range(h)]


def decode(code: int, scale: int):
    """Exact value of a 4-bit code under an E8M0 scale byte (None for the NaN scale)."""
    if scale == 0xFF:
        return None
    m = E2M1_GRID[code & 7] * Fraction(2) ** (scale - 127)
    return -m if code & 8 else m


def gemm_exact(codes_a, scales_a, codes_b, scales_b, alpha=Fraction(1)):
    """C[m][n] = alpha sum_k deq(A)[m][k] deq(B)[n][k] with unpacked codes (lists of lists,
    one code per element) and per-32 scales; exact Fractions (None where a scale is 0xFF)."""
    M, K = len(codes_a), len(codes_a[0])
    N = len(codes_b)
    out = []
    for m in range(M):
        row = []
        for n in range(N):
            acc = Fraction(0)
            nan = False
            for k in range(K):
                a = decode(codes_a[m][k], scales_a[m][k // 32])
                b = decode(codes_b[n][k], scales_b[n][k // 32])
                if a is None or b is None:
                    nan = True
                    break
                acc += a * b
            row.append(None if nan else alpha * acc)
        out.append(row)
    return out


PHILOX_CONSTANTS = {
    # multipliers (M0, M1) and key increments (W0, W1) per word width
    32: (0xD2511F53, 0xCD9E8D57, 0x9E3779B9, 0xBB67AE85),
    64: (0xD2E7470EE14C6C93, 0xCA5A826395121157, 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B),
}


def philox(counter, key, width=32, rounds=10):
    """Philox4xW-R block function, generic in the word width W."""
    M0, M1, W0, W1 = PHILOX_CONSTANTS[width]
    mask = (1 << width) - 1
    x = [int(c) & mask for c in counter]
    k = [int(c) & mask for c in key]
    for r in range(rounds):
        if r:
            k = [(k[0] + W0) & mask, (k[1] + W1) & mask]
        p0 = M0 * x[0]
        p1 = M1 * x[2]
        x = [(p1 >> width) ^ x[1] ^ k[0], p1 & mask, (p0 >> width) ^ x[3] ^ k[1], p0 & mask]
    return x


def weyl_constant(width: int, which: str) -> int:
    """floor(2^W * frac) for the golden ratio's fractional part ('phi') or sqrt(3) - 1 ('sqrt3'),
    computed with exact integer square roots."""
    s = 1 << (2 * width + 8)   # extra guard bits
    if which == "phi":   # (sqrt(5) - 1) / 2
        v = (math.isqrt(5 * s * s) - s) // 2
    elif which == "sqrt3":
        v = math.isqrt(3 * s * s) - s
    else:
        raise ValueError(which)
    return (v << width) // s


def sr_word(seed: int, stream: int, index: int) -> int:
    """Random word for the element with quantized-layout index ``index``."""
    c = index >> 2
    out = philox([c & 0xFFFFFFFF, c >> 32, stream & 0xFFFFFFFF, 0],
                  [seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], 32)
    return out[index & 3]

/*
 * CPU oracle for MXFP4 quantization behind a block Hadamard rotation, and for the
 * block-scaled FP4 GEMM that consumes it.
 *
 * TEST INFRASTRUCTURE ONLY. This file is slow on purpose and shares no code, header, table
 * or constant with the HIP library. Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may build, load or call it. The product path never does.
 *
 * What it computes (sources):
 *  - The method: gist.science summary of "MXFP4 LLM pretraining" (Llama-3.1-8B on MI355X),
 *    section "방법론" (Methodology): every GEMM of the linear layer -- forward (Fprop), activation
 *    gradient (Dgrad) and weight gradient (Wgrad) -- runs in MXFP4; the stabilisers tried are
 *    stochastic rounding, randomized Hadamard and deterministic 16x16 / 32x32 Hadamard rotations;
 *    section "주요 기여 및 발견" §2: the deterministic H16 applied to the whole pipeline is the
 *    one that restores convergence. The rotation comes before quantization.
 *  - The number format: OCP Microscaling Formats (MX) v1.0, MXFP4 = blocks of 32 E2M1 elements
 *    sharing one E8M0 scale; shared exponent = floor(log2(block amax)) - emax(E2M1) with
 *    emax = 2; elements converted with round-to-nearest-even and saturation.
 *    Two 4-bit codes per byte: molayo1419.me NVFP4 article, section "주요 사실" (key facts).
 *  - Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 *    SC'11 (the round function, multipliers and Weyl key increments as published there).
 *
 * Readings where the pages are silent (all fixed here, and identically in the HIP path):
 *  - H_h is the unnormalised Sylvester Hadamard, H[i][j] = (-1)^popcount(i & j), applied to each
 *    aligned group of h consecutive elements along the quantization axis. It is computed as a
 *    fast Walsh-Hadamard transform in IEEE binary32 with round-to-nearest-even, stages of stride
 *    1, 2, 4, ... and the pair update (u, w) -> (u + w, u - w). The quantized code is decided in
 *    this precision because the kernel decides it in this precision.
 *  - amax over a block of 32 rotated values; any NaN or infinity makes the scale byte 0xFF and
 *    every code of that block 0. An all-zero block gets scale byte 0.
 *  - Code nibble: bit 3 = sign of the rotated value (also for -0 and values that round to 0),
 *    bits 2..0 = magnitude index into {0, 0.5, 1, 1.5, 2, 3, 4, 6}. Even element -> low nibble.
 *  - Stochastic rounding: |v| >= 6 saturates to 6; otherwise with lo <= |v| < hi the two
 *    neighbouring grid values and f = (|v| - lo) / (hi - lo), the magnitude rounds up iff
 *    floor(r / 2^10) < floor(f * 2^22), r being a 32-bit Philox word: 22 random bits against
 *    the fractional position truncated to 22 bits, so P(up) = floor(f 2^22) / 2^22 (the rule
 *    gfx950's stochastic FP4 conversion applies). Key = (seed mod 2^32, seed >> 32); for the
 *    element at position j of quantized row o (index i = o * L + j, L the quantized length),
 *    counter = (floor(i/4) mod 2^32, floor(i/4) >> 32, stream, 0), word i mod 4.
 *  - Scale variant "no clip" (rounding argument | 0x10): the smallest scale that maps the block
 *    maximum to at most 6, i.e. S + 1 exactly when amax > 6 * 2^(S - 127); no element saturates.
 *  - Randomized Hadamard (the pages name it as the other rotation tried, without a construction):
 *    y = H_h (d .* x) per aligned group, with d_j = -1 or +1 for position j along the quantized
 *    axis -- the same for every quantized row, so two operands rotated with the same key keep
 *    their product up to h. d_j = -1 iff bit (j mod 32) of word ((j / 32) mod 4) of
 *    Philox4x32-10 with key (seed mod 2^32, seed >> 32) and counter (floor(j/128) mod 2^32,
 *    floor(j/128) >> 32, 0, 1) is set (the last counter word 1 keeps it apart from the
 *    stochastic-rounding words, whose last counter word is 0).
 *  - Orthonormal rotation (hadamard | 0x200; the pages name the 16x16 and 32x32 matrices without
 *    a normalisation): y = H_h x / sqrt(h), computed as the binary32 transform above followed by
 *    one binary32 multiplication of every value by the binary32 number nearest to 1/sqrt(h)
 *    (0.25 for h = 16, exact; 2^-2.5 rounded for h = 32). A product of two such operands needs no
 *    1/h factor.
 *  - GEMM: C[m][n] = alpha * sum_k deq(A)[m][k] * deq(B)[n][k]; each 32-element block product is
 *    an exact integer sum, scaled exactly, and blocks are summed in binary64.
 *
 * Pins (tests/test_oracle_pins.py, no GPU): the E2M1 value table and nearest-even tie points,
 * the scale rule's closed form, the Hadamard matrix and its identities, round-trip bounds,
 * exact constructions and rational brute force for the GEMM and both roundings, the published
 * Philox4x32-10 known-answer vectors, and the stochastic rounding's word choice and key through
 * the published zero-counter block (elements 0..3 of row 0 under seed 0, stream 0 decide with its
 * four words). Parity unpinned: the conventions the pages leave open and that no outside fact can
 * fix -- the sign bit of zero codes, the nibble order, which counter words carry the index's high
 * bits and the stream (zero in the published block), and the sign sequence of the randomized
 * rotation (its use, signs then H, is pinned by an exact construction). Only agreement between
 * this oracle and the GPU checks them.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fno-fast-math -shared -fPIC (see build.py).
 * OpenMP splits only the outermost loop over independent rows; per-row arithmetic is sequential.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- E2M1 / E8M0 -------------- */

/* Magnitude of an E2M1 code's low three bits: 2 exponent bits (bias 1), 1 mantissa bit;
 * exponent field 0 is subnormal (0 or 0.5). */
static double e2m1_magnitude(unsigned mag3)
{
    unsigned e = (mag3 >> 1) & 3u, m = mag3 & 1u;
    if (e == 0) return 0.5 * (double)m;
    return ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
}

/* Index of an exactly representable E2M1 magnitude. */
static unsigned e2m1_index(double mag)
{
    for (unsigned i = 0; i < 8; ++i)
        if (e2m1_magnitude(i) == mag) return i;
    abort(); /* unreachable: callers only pass grid values */
}

/* Spacing of the E2M1 grid around magnitude a (0 <= a < 6): 0.5 below 2, 1 in [2,4), 2 in [4,6]. */
static double e2m1_quantum(double a)
{
    if (a < 2.0) return 0.5;
    if (a < 4.0) return 1.0;
    return 2.0;
}

/* Round-to-nearest, ties to the even code, saturating at 6 (IEEE-style conversion to a format
 * whose largest finite value is 6 and which has no infinity). a = |v| >= 0. Returns 3-bit index. */
static unsigned e2m1_round_nearest_even(double a)
{
    if (a >= 6.0) return 7;
    double q = e2m1_quantum(a);
    double n = a / q; /* exact: q is a power of two */
    double fl = floor(n);
    double frac = n - fl;
    double k = fl;
    /* even multiple of the quantum <-> even code (mantissa bit 0) */
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) k = fl + 1.0;
    return e2m1_index(k * q);
}

/* Stochastic rounding of a = |v| >= 0 with one 32-bit random word r: the fractional position f
 * of a between its two grid neighbours, truncated to 22 bits, against the top 22 bits of r. */
static unsigned e2m1_round_stochastic(double a, uint32_t r)
{
    if (a >= 6.0) return 7;
    double q = e2m1_quantum(a);
    double n = a / q;
    double lo = floor(n);
    double f22 = floor(ldexp(n - lo, 22));  /* floor(f * 2^22), exact */
    double k = ((double)(r >> 10) < f22) ? lo + 1.0 : lo;
    return e2m1_index(k * q);
}

/* E8M0 shared scale byte from the block amax (binary64, exact copy of a binary32 value).
 * OCP MX: shared exponent = floor(log2(amax)) - 2, clamped to the E8M0 range [-127, 127]. */
static unsigned e8m0_from_amax(double amax, int nonfinite)
{
    if (nonfinite) return 0xFFu;
    if (amax == 0.0) return 0u;
    int e;
    (void)frexp(amax, &e);         /* amax = m * 2^e, m in [0.5, 1) -> floor(log2 amax) = e - 1 */
    int shared = (e - 1) - 2;
    if (shared < -127) shared = -127;
    if (shared > 127) shared = 127;
    return (unsigned)(shared + 127);
}

/* The no-clip variant of the scale: the smallest scale byte, from S upward, that maps the block
 * maximum to at most 6 (the largest E2M1 magnitude), so that no element of the block
 * saturates. ldexp of 6 by a power of two is exact. */
static unsigned e8m0_noclip(double amax, unsigned S)
{
    if (S == 0xFFu || amax == 0.0) return S;
    while (S < 254u && amax > ldexp(6.0, (int)S - 127)) ++S;
    return S;
}

/* ---------------------------------------------------------------- Philox4x32-10 ------------- */

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;     /* round multipliers */
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;     /* key increments */
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) { k0 += W0; k1 += W1; }
        uint64_t p0 = (uint64_t)M0 * (uint64_t)x0;
        uint64_t p1 = (uint64_t)M1 * (uint64_t)x2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t y0 = hi1 ^ x1 ^ k0;
        uint32_t y1 = lo1;
        uint32_t y2 = hi0 ^ x3 ^ k1;
        uint32_t y3 = lo0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* The random word for element index i under (seed, stream). */
static uint32_t sr_word(uint64_t seed, uint32_t stream, uint64_t i)
{
    uint64_t c = i >> 2;
    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), stream, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[i & 3u];
}

/* Sign of the randomized-Hadamard diagonal at position j along the quantized axis: 1 = negate. */
static int rht_negate(uint64_t seed, uint64_t j)
{
    uint64_t c = j >> 7;
    uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), 0u, 1u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (int)((out[(j >> 5) & 3u] >> (j & 31u)) & 1u);
}

/* d_j for j = 0 .. count - 1 as +1 / -1 bytes. */
void oracle_rht_signs(uint64_t seed, int64_t count, int8_t *out)
{
    for (int64_t j = 0; j < count; ++j) out[j] = rht_negate(seed, (uint64_t)j) ? (int8_t)-1 : (int8_t)1;
}

/* ---------------------------------------------------------------- Hadamard ------------------ */

/* In-place unnormalised Walsh-Hadamard transform of h values in binary32 (h a power of two). */
static void fwht_binary32(float *v, int h)
{
    for (int s = 1; s < h; s <<= 1)
        for (int i = 0; i < h; ++i)
            if ((i & s) == 0) {
                float u = v[i], w = v[i + s];
                v[i] = u + w;
                v[i + s] = u - w;
            }
}

void oracle_fwht_binary32(float *v, int64_t count, int h)
{
    for (int64_t g = 0; g + h <= count; g += h) fwht_binary32(v + g, h);
}

/* ---------------------------------------------------------------- quantize ------------------ */

static float load_element(const void *x, int dtype, int64_t r, int64_t c, int64_t ldx)
{
    if (dtype == 0) { /* bfloat16: the upper half of a binary32 */
        uint16_t b = ((const uint16_t *)x)[r * ldx + c];
        uint32_t bits = (uint32_t)b << 16;
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    return ((const float *)x)[r * ldx + c];
}

/*
 * Quantize T[rows][cols] (row stride ldx elements; dtype 0 = bf16, 1 = f32).
 * axis = 1: along each row (L = cols), outputs q[rows][cols/2], scales[rows][cols/32].
 * axis = 0: along each column (L = rows), outputs the quantized transpose q[cols][rows/2],
 *           scales[cols][rows/32].
 * h in {0, 16, 32}, or 16 / 32 plus 0x100 for the randomized Hadamard (signs keyed by seed)
 * and / or plus 0x200 for the orthonormal scaling H_h / sqrt(h);
 * rounding 0 = nearest-even, 1 = stochastic (Philox), plus 0x10 for the no-clip scale.
 * Returns 0 on success.
 */
int oracle_quantize(const void *x, int dtype, int64_t rows, int64_t cols, int64_t ldx, int axis,
                    int h, int rounding, uint64_t seed, uint32_t stream, uint8_t *q, uint8_t *scales)
{
    const int64_t L = axis ? cols : rows;
    const int64_t outer = axis ? rows : cols;
    const int randomized = (h & 0x100) != 0;
    const int orthonormal = (h & 0x200) != 0;
    const int noclip = (rounding & 0x10) != 0;
    h &= ~0x300;
    rounding &= ~0x10;
    if (L % 32 != 0 || (h != 0 && h != 16 && h != 32) || (axis != 0 && axis != 1)) return 1;
    if ((randomized || orthonormal) && h == 0) return 1;
    /* binary32 nearest to 1/sqrt(h): sqrt and division are correctly rounded in binary64, and
     * 1/sqrt(h) is nowhere near a binary32 rounding boundary for h = 16, 32 */
    const float norm = orthonormal ? (float)(1.0 / sqrt((double)h)) : 1.0f;
    int status = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t o = 0; o < outer; ++o) {
        float *y = (float *)malloc(sizeof(float) * (size_t)(L > 0 ? L : 1));
        if (!y) { status = 2; continue; }
        for (int64_t j = 0; j < L; ++j)
            y[j] = axis ? load_element(x, dtype, o, j, ldx) : load_element(x, dtype, j, o, ldx);
        if (randomized)
            for (int64_t j = 0; j < L; ++j)
                if (rht_negate(seed, (uint64_t)j)) y[j] = -y[j];  /* exact */
        if (h) oracle_fwht_binary32(y, L, h);
        if (orthonormal)
            for (int64_t j = 0; j < L; ++j) y[j] = y[j] * norm; /* one binary32 multiply */
        for (int64_t b = 0; b < L / 32; ++b) {
            const float *blk = y + 32 * b;
            double amax = 0.0;
            int nonfinite = 0;
            for (int t = 0; t < 32; ++t) {
                if (!isfinite(blk[t])) nonfinite = 1;
                else if (fabs((double)blk[t]) > amax) amax = fabs((double)blk[t]);
            }
            unsigned S = e8m0_from_amax(amax, nonfinite);
            if (noclip) S = e8m0_noclip(amax, S);
            scales[o * (L / 32) + b] = (uint8_t)S;
            for (int t = 0; t < 32; ++t) {
                unsigned code = 0;
                if (S != 0xFFu) {
                    double v = ldexp((double)blk[t], 127 - (int)S); /* exact */
                    unsigned mag;
                    if (rounding == 0) {
                        mag = e2m1_round_nearest_even(fabs(v));
                    } else {
                        uint64_t idx = (uint64_t)o * (uint64_t)L + (uint64_t)(32 * b + t);
                        mag = e2m1_round_stochastic(fabs(v), sr_word(seed, stream, idx));
                    }
                    code = (signbit(blk[t]) ? 8u : 0u) | mag;
                }
                int64_t j = 32 * b + t;
                uint8_t *dst = q + o * (L / 2) + j / 2;
                if ((j & 1) == 0) *dst = (uint8_t)code;
                else *dst = (uint8_t)(*dst | (code << 4));
            }
        }
        free(y);
    }
    return status;
}

/* ---------------------------------------------------------------- dequantize ---------------- */

static double decode_code(unsigned code)
{
    double m = e2m1_magnitude(code & 7u);
    return (code & 8u) ? -m : m;
}

/* out[o][j] = decoded value, binary64; scale 0xFF gives NaN. */
void oracle_dequantize(const uint8_t *q, const uint8_t *scales, int64_t outer, int64_t L, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t o = 0; o < outer; ++o)
        for (int64_t j = 0; j < L; ++j) {
            unsigned S = scales[o * (L / 32) + j / 32];
            uint8_t byte = q[o * (L / 2) + j / 2];
            unsigned code = (j & 1) ? (byte >> 4) : (byte & 15u);
            out[o * L + j] = (S == 0xFFu) ? NAN : ldexp(decode_code(code), (int)S - 127);
        }
}

/* ---------------------------------------------------------------- GEMM ---------------------- */

/* Twice the E2M1 value of a code: an integer in [-12, 12]. */
static int twice_value(unsigned code)
{
    int m = (int)(2.0 * e2m1_magnitude(code & 7u));
    return (code & 8u) ? -m : m;
}

static unsigned code_at(const uint8_t *q, int64_t row, int64_t K, int64_t k)
{
    uint8_t byte = q[row * (K / 2) + k / 2];
    return (k & 1) ? (unsigned)(byte >> 4) : (unsigned)(byte & 15u);
}

/* One output: value and the tolerance basis sum_k |deqA[m][k] * deqB[n][k]| (both times alpha). */
static void gemm_one(const uint8_t *aq, const uint8_t *as, const uint8_t *bq, const uint8_t *bs,
                     int64_t m, int64_t n, int64_t K, double alpha, double *val, double *absval)
{
    double acc = 0.0, acc_abs = 0.0;
    int nan = 0;
    for (int64_t b = 0; b < K / 32; ++b) {
        unsigned sa = as[m * (K / 32) + b], sb = bs[n * (K / 32) + b];
        if (sa == 0xFFu || sb == 0xFFu) { nan = 1; continue; }
        long dot = 0, adot = 0;
        for (int64_t t = 0; t < 32; ++t) {
            int64_t k = 32 * b + t;
            long p = (long)twice_value(code_at(aq, m, K, k)) * (long)twice_value(code_at(bq, n, K, k));
            dot += p;
            adot += labs(p);
        }
        /* (2a)(2b) = 4ab; scales 2^(sa-127) * 2^(sb-127) */
        acc += ldexp((double)dot, (int)sa + (int)sb - 254 - 2);
        acc_abs += ldexp((double)adot, (int)sa + (int)sb - 254 - 2);
    }
    *val = nan ? NAN : alpha * acc;
    if (absval) *absval = fabs(alpha) * acc_abs;
}

/* C[M][N] (binary64) = alpha * deq(A)[M][K] . deq(B)[N][K]^T. cabs (optional) gets the
 * per-output tolerance basis. */
void oracle_gemm(const uint8_t *aq, const uint8_t *as, const uint8_t *bq, const uint8_t *bs,
                 int64_t M, int64_t N, int64_t K, double alpha, double *c, double *cabs)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            gemm_one(aq, as, bq, bs, m, n, K, alpha, &c[m * N + n], cabs ? &cabs[m * N + n] : NULL);
}

/* The same for a list of (m, n) pairs. */
void oracle_gemm_sampled(const uint8_t *aq, const uint8_t *as, const uint8_t *bq, const uint8_t *bs,
                         int64_t K, double alpha, const int64_t *ms, const int64_t *ns, int64_t count,
                         double *c, double *cabs)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < count; ++i)
        gemm_one(aq, as, bq, bs, ms[i], ns[i], K, alpha, &c[i], cabs ? &cabs[i] : NULL);
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

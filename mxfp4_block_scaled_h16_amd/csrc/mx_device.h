// Device-side building blocks of the MXFP4 quantizers (gfx950).
//
// Format: OCP Microscaling Formats v1.0 MXFP4 -- 32-element blocks, one E8M0 scale byte per
// block, E2M1 elements {0, .5, 1, 1.5, 2, 3, 4, 6} with a sign bit, two per byte (even element in
// the low nibble). The rotation is the deterministic block Hadamard of the gist.science summary of
// "MXFP4 LLM pretraining", section 방법론 (Methodology, H16 / H32), applied before quantization.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------- input widening --

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// ---------------------------------------------------------------------------- magnitudes ------
// |x| as an unsigned bit pattern orders like |x|, with NaN above +inf.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

// largest |v[i]| of N values as a bit pattern
template <int N>
__device__ __forceinline__ uint32_t amax_bits(const float *v)
{
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) m = max(m, abs_bits(v[i]));
    return m;
}

// The largest |x * norm| from the largest |x| (bit pattern amax): binary32 multiplication by a
// positive number is monotonic in |x|, so scaling the maximum gives the maximum of the scaled.
__device__ __forceinline__ uint32_t scaled_amax(uint32_t amax, float norm)
{
    return abs_bits(__uint_as_float(amax) * norm);
}

// ---------------------------------------------------------------------------- block Hadamard --
// Unnormalised Sylvester transform of n values held in registers, binary32, strides 1, 2, 4, ...,
// pair update (u, w) -> (u + w, u - w). The upper element is always u - w (never -(w - u)) so
// signed zeros come out the same in every implementation of this order.
template <int N>
__device__ __forceinline__ void fwht_regs(float *v)
{
#pragma unroll
    for (int s = 1; s < N; s <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if ((i & s) == 0) {
                const float u = v[i], w = v[i + s];
                v[i] = u + w;
                v[i + s] = u - w;
            }
        }
    }
}

// fwht_regs<N> that also returns the largest |output| as a binary32 bit pattern. In the last
// stage the larger of |u + w| and |u - w| is |u| + |w|, and binary32 rounding is monotonic and
// symmetric, so the larger of the two rounded outputs' magnitudes is the rounded |u| + |w|: one
// add with absolute-value operands per output pair instead of two masks and a max. A NaN or
// infinity among the outputs gives a pattern >= 0x7F800000 here as well (infinity minus infinity
// becomes infinity instead of NaN), which is all the scale rule looks at.
template <int N>
__device__ __forceinline__ uint32_t fwht_regs_amax(float *v)
{
#pragma unroll
    for (int s = 1; s < N / 2; s <<= 1) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            if ((i & s) == 0) {
                const float u = v[i], w = v[i + s];
                v[i] = u + w;
                v[i + s] = u - w;
            }
        }
    }
    uint32_t m = 0u;
    constexpr int s = N / 2;
#pragma unroll
    for (int i = 0; i < s; ++i) {
        const float u = v[i], w = v[i + s];
        v[i] = u + w;
        v[i + s] = u - w;
        m = max(m, __float_as_uint(fabsf(u) + fabsf(w)));
    }
    return m;
}

// Rotate 32 values that form one MX block: H in {0, 16, 32}.
template <int H>
__device__ __forceinline__ void rotate_block(float *v)
{
    if constexpr (H == 16) {
        fwht_regs<16>(v);
        fwht_regs<16>(v + 16);
    } else if constexpr (H == 32) {
        fwht_regs<32>(v);
    }
}

// Rotate the 32 values of one MX block (H in {0, 16, 32}, as rotate_block) and return their
// largest magnitude as a bit pattern.
template <int H>
__device__ __forceinline__ uint32_t rotate_block_amax(float *v)
{
    if constexpr (H == 16) {
        const uint32_t a = fwht_regs_amax<16>(v);
        const uint32_t b = fwht_regs_amax<16>(v + 16);
        return max(a, b);
    } else if constexpr (H == 32) {
        return fwht_regs_amax<32>(v);
    } else {
        return amax_bits<32>(v);
    }
}

// v[i] *= s in binary32 (the orthonormal rotation's 1/sqrt(h), after the transform)
template <int N>
__device__ __forceinline__ void scale_values(float *v, float s)
{
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = v[i] * s;
}

// ---------------------------------------------------------------------------- scale -----------
// E8M0 byte from the block's largest |value| bit pattern: biased exponent E of amax gives
// floor(log2 amax) = E - 127, so the shared exponent E - 127 - 2 is the byte E - 2 (clamped at 0).
__device__ __forceinline__ uint32_t e8m0_from_amax_bits(uint32_t amax_bits)
{
    if (amax_bits >= 0x7F800000u) return 0xFFu;
    const uint32_t e = amax_bits >> 23;
    return e > 2u ? e - 2u : 0u;
}

// The no-clip variant: one more when the block maximum maps above 6 under S = max(E - 2, 0),
// i.e. E >= 2 and the amax significand above 1.5 (then S + 1 maps it into (3, 4)).
__device__ __forceinline__ uint32_t e8m0_noclip(uint32_t amax_bits, uint32_t s)
{
    const bool up = s != 0xFFu && (amax_bits >> 23) >= 2u && (amax_bits & 0x7FFFFFu) > 0x400000u;
    return s + (up ? 1u : 0u);
}

// ---------------------------------------------------------------------------- E2M1 encode -----
// Nearest-even encoding uses gfx950's v_cvt_scalef32_pk_fp4_f32, which converts two binary32
// values divided by a binary32 scale to two E2M1 codes (first value in the low nibble) with
// ties to the even code, saturation at 6 and the sign bit of the scaled value kept for zero
// results -- the encoding defined above. Dividing by 2^(S - 127) is exact for S in [1, 252]
// (every finite block has S <= 252); an S = 0 block is pre-multiplied by 2 and divided by
// 2^-126 so the scale operand never is a subnormal.

// binary32 divisor 2^(S - 127) for S in [1, 252] (exponent field S, zero mantissa)
__device__ __forceinline__ float e8m0_divisor(uint32_t s) { return __uint_as_float((s > 1u ? s : 1u) << 23); }

// Codes of 8 consecutive values (scaled by 2^(127 - S)) as one word, element k in nibble k.
__device__ __forceinline__ uint32_t encode8_nearest(const float *v, float divisor)
{
    uint32_t w = 0u;
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], divisor, 0);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], divisor, 1);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], divisor, 2);
    w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], divisor, 3);
    return w;
}

// The S = 0 case of the divisor rule above: double every value of the block (exact).
template <int N>
__device__ __forceinline__ void prescale_if_zero_scale(float *v, uint32_t s)
{
    if (s == 0u) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] *= 2.0f;
    }
}

// ---------------------------------------------------------------------------- Philox4x32-10 --
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds;
// each multiplies words 0 and 2 by fixed odd constants, swaps the halves of the products in and
// mixes in the other words and the round key; the key advances by fixed Weyl increments.
struct Philox4 {
    uint32_t w[4];
};

// One round; TT is the truth table of the three-input XORs (0x96), or of their complement (0x69).
template <int TT>
__device__ __forceinline__ void philox_round(uint32_t &c0, uint32_t &c1, uint32_t &c2, uint32_t &c3,
                                             uint32_t k0, uint32_t k1)
{
    const uint64_t p = (uint64_t)0xD2511F53u * c0;
    const uint64_t q = (uint64_t)0xCD9E8D57u * c2;
    // three-input XORs in one gfx950 bitop3 instruction each
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(q >> 32), c1, k0, TT);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p >> 32), c3, k1, TT);
    c1 = (uint32_t)q;
    c3 = (uint32_t)p;
    c0 = n0;
    c2 = n2;
}

// COMPLEMENT returns the bitwise complement of the four words; words 0 and 2 get it for free
// from the last round's three-input XORs.
template <bool COMPLEMENT = false>
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 9; ++round) {
        philox_round<0x96>(c0, c1, c2, c3, k0, k1);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    philox_round<COMPLEMENT ? 0x69 : 0x96>(c0, c1, c2, c3, k0, k1);
    Philox4 r;
    r.w[0] = c0;
    r.w[1] = COMPLEMENT ? ~c1 : c1;
    r.w[2] = c2;
    r.w[3] = COMPLEMENT ? ~c3 : c3;
    return r;
}

// NB consecutive Philox4x32-10 blocks, counters (c + b, c >> 32, stream_id, 0) for b < NB, with
// c a multiple of NB (so c + b never carries into counter word 1). Counter words 1-3 are the same
// for every block, and so are two of the first rounds' products: round 1 multiplies word 2 (the
// stream) and round 2 multiplies word 0 (which round 1 made from words 1 and 2 and the key only).
// Those two 64-bit multiply-adds are formed once, leaving 18 of 20 per block. COMPLEMENT as for
// philox4x32_10.
template <int NB, bool COMPLEMENT>
__device__ __forceinline__ void philox4x32_10_run(uint64_t c, uint32_t stream_id, uint32_t k0, uint32_t k1,
                                                  Philox4 (&out)[NB])
{
    const uint32_t c_lo = (uint32_t)c, c_hi = (uint32_t)(c >> 32);
    // round 1, shared part: word 2's product; the new words 0 and 1
    const uint64_t q1 = (uint64_t)0xCD9E8D57u * stream_id;
    const uint32_t w0_1 = __builtin_amdgcn_bitop3_b32((uint32_t)(q1 >> 32), c_hi, k0, 0x96);
    const uint32_t w1_1 = (uint32_t)q1;
    // round 2, shared part: word 0's product
    const uint32_t k0_2 = k0 + 0x9E3779B9u, k1_2 = k1 + 0xBB67AE85u;
    const uint64_t p2 = (uint64_t)0xD2511F53u * w0_1;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        // round 1, per block: word 0's product (word 3 of the counter is 0)
        const uint64_t p1 = (uint64_t)0xD2511F53u * (c_lo + (uint32_t)b);
        const uint32_t w2_1 = (uint32_t)(p1 >> 32) ^ k1;
        const uint32_t w3_1 = (uint32_t)p1;
        // round 2, per block: word 2's product
        const uint64_t q2 = (uint64_t)0xCD9E8D57u * w2_1;
        uint32_t x0 = __builtin_amdgcn_bitop3_b32((uint32_t)(q2 >> 32), w1_1, k0_2, 0x96);
        uint32_t x2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p2 >> 32), w3_1, k1_2, 0x96);
        uint32_t x1 = (uint32_t)q2;
        uint32_t x3 = (uint32_t)p2;
        // rounds 3-10
        uint32_t kk0 = k0_2 + 0x9E3779B9u, kk1 = k1_2 + 0xBB67AE85u;
#pragma unroll
        for (int round = 2; round < 9; ++round) {
            philox_round<0x96>(x0, x1, x2, x3, kk0, kk1);
            kk0 += 0x9E3779B9u;
            kk1 += 0xBB67AE85u;
        }
        philox_round<COMPLEMENT ? 0x69 : 0x96>(x0, x1, x2, x3, kk0, kk1);
        out[b].w[0] = x0;
        out[b].w[1] = COMPLEMENT ? ~x1 : x1;
        out[b].w[2] = x2;
        out[b].w[3] = COMPLEMENT ? ~x3 : x3;
    }
}

// ---------------------------------------------------------------- randomized Hadamard -------
// Sign diagonal of the randomized rotation y = H (d .* x): bit t of the returned word is set iff
// position 32 c + t along the quantized axis is negated. Word c % 4 of the Philox4x32-10 block
// with counter (c / 4 mod 2^32, c / 4 >> 32, 0, 1): the last counter word 1 keeps these words
// apart from the stochastic-rounding words (last counter word 0) under the same key.
__device__ __forceinline__ uint32_t rht_sign_word(uint64_t c, uint32_t key0, uint32_t key1)
{
    const uint64_t b = c >> 2;
    const Philox4 r = philox4x32_10((uint32_t)b, (uint32_t)(b >> 32), 0u, 1u, key0, key1);
    const uint32_t w = (uint32_t)c & 3u;
    return w == 0u ? r.w[0] : (w == 1u ? r.w[1] : (w == 2u ? r.w[2] : r.w[3]));
}

// Negate v[e] where bit e of `bits` is set (an exact sign-bit flip).
template <int N>
__device__ __forceinline__ void apply_signs(float *v, uint32_t bits)
{
#pragma unroll
    for (int e = 0; e < N; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) ^ (((bits >> e) & 1u) << 31));
}

// ---------------------------------------------------------------------------- stochastic -----
// Stochastic codes of 8 consecutive values y[0..7] (block scale byte S, values already
// pre-doubled when S = 0, divisor = e8m0_divisor(S)) whose first element has position index0 (a
// multiple of 8) in the quantized output: element 4 b + k draws word k of Philox block
// (index0 / 4 + b).
//
// gfx950's v_cvt_scalef32_sr_pk_fp4_f32 divides a pair of binary32 values by the scale and
// rounds each to E2M1 stochastically, saturating at 6 and keeping the sign of the value (also
// for zero results). For the first value of the pair and random operand u it rounds the
// magnitude up iff u plus the value's fractional position between its two grid neighbours,
// truncated to 22 bits and aligned to the top of the word, carries out of 32 bits; with
// u = ~r that is floor(r / 2^10) < floor(2^22 f), the rounding rule defined above. The second
// value of a pair would draw from a shifted copy of the same operand, so each instruction
// converts one element, with partner 0.0 (which encodes as +0 and never rounds up): byte 0 of
// the result holds the element's code in its low nibble and 0 above it. Only that byte is
// defined (the compiler does not carry the other bytes of the destination through), so pairs
// are merged with a shift and the four valid bytes gathered with byte permutes.

// the code of y in bits 0-3 and 0 in bits 4-7 (bits 8-31 undefined), given nr = ~r
__device__ __forceinline__ uint32_t sr_fp4_byte0(float y, uint32_t nr, float divisor)
{
    const f32x2 pair = {y, 0.0f};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, pair, nr, divisor, 0);
}

// The same from the complemented words (~r) of the two blocks, r0 for elements 0-3 and r1 for 4-7.
__device__ __forceinline__ uint32_t encode8_sr_words(const float *y, float divisor, const Philox4 &r0,
                                                     const Philox4 &r1)
{
    // byte 0 of p_k = codes of elements 2k (low nibble) and 2k + 1 (high nibble)
    const uint32_t p0 = (sr_fp4_byte0(y[1], r0.w[1], divisor) << 4) | sr_fp4_byte0(y[0], r0.w[0], divisor);
    const uint32_t p1 = (sr_fp4_byte0(y[3], r0.w[3], divisor) << 4) | sr_fp4_byte0(y[2], r0.w[2], divisor);
    const uint32_t p2 = (sr_fp4_byte0(y[5], r1.w[1], divisor) << 4) | sr_fp4_byte0(y[4], r1.w[0], divisor);
    const uint32_t p3 = (sr_fp4_byte0(y[7], r1.w[3], divisor) << 4) | sr_fp4_byte0(y[6], r1.w[2], divisor);
    // v_perm_b32(hi, lo, sel): selector byte 0-3 picks that byte of lo, 4-7 of hi, 0x0c gives 0
    const uint32_t q01 = __builtin_amdgcn_perm(p1, p0, 0x0C0C0400u);  // [p0.b0, p1.b0, 0, 0]
    const uint32_t q23 = __builtin_amdgcn_perm(p3, p2, 0x04000C0Cu);  // [0, 0, p2.b0, p3.b0]
    return q01 | q23;
}

// Stochastic codes of W * 8 consecutive values (index0 a multiple of 4 W): word w of the result
// holds values 8 w .. 8 w + 7, from the 2 W Philox blocks formed as one run.
template <int W>
__device__ __forceinline__ void encode_stochastic(const float *y, float divisor, uint64_t index0, uint32_t key0,
                                                  uint32_t key1, uint32_t stream_id, uint32_t (&words)[W])
{
    Philox4 r[2 * W];
    philox4x32_10_run<2 * W, true>(index0 >> 2, stream_id, key0, key1, r);
#pragma unroll
    for (int w = 0; w < W; ++w) words[w] = encode8_sr_words(y + 8 * w, divisor, r[2 * w], r[2 * w + 1]);
}

// ---------------------------------------------------------------------------- cross-lane ------
// Value of lane (l ^ X) for X in {1, 2} (DPP quad permutation; every lane must be active).
template <int X>
__device__ __forceinline__ uint32_t quad_xor(uint32_t v)
{
    static_assert(X == 1 || X == 2, "quad xor");
    constexpr int ctrl = X == 1 ? 0xB1 : 0x4E;  // quad_perm [1,0,3,2] / [2,3,0,1]
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, true);
}

// One Walsh-Hadamard stage whose pairs straddle lanes l and l ^ X (each lane holds N values,
// the lane with bit X set holds the higher-index element of every pair): the lower lane keeps
// u + w, the upper lane u - w, computed as u + (-w) (IEEE subtraction), so the results are
// bit-identical to the in-register stage.
template <int X, int N = 8>
__device__ __forceinline__ void fwht_cross_stage(float *v, bool upper)
{
    const uint32_t flip = upper ? 0x80000000u : 0u;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float other = __uint_as_float(quad_xor<X>(__float_as_uint(v[i])));
        v[i] = other + __uint_as_float(__float_as_uint(v[i]) ^ flip);
    }
}

}  // namespace mx

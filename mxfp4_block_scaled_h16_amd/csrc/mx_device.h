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

// v[i] *= s in binary32 (the orthonormal rotation's 1/sqrt(h), after the transform)
template <int N>
__device__ __forceinline__ void scale_values(float *v, float s)
{
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = v[i] * s;
}

// ---------------------------------------------------------------------------- scale -----------
// |x| as an unsigned bit pattern orders like |x|, with NaN above +inf.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }

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

// 2^(127 - S) as binary32 multiplier for S in [0, 253] (exponent field 254 - S in [1, 254]).
__device__ __forceinline__ float e8m0_reciprocal(uint32_t s)
{
    const uint32_t sc = s < 253u ? s : 253u;
    return __uint_as_float((254u - sc) << 23);
}

// Stochastic E2M1 magnitude index of a = |v| >= 0 with random word r: saturate at 6, else round
// up to the next grid value iff r < 2^32 f, f = fractional position of a between its two grid
// neighbours. a is first clamped to 6 (6 is its own lower neighbour, index 7, with f = 0, so
// everything from 6 up saturates; a NaN also lands there, in a block whose codes are discarded).
// Then, from the bit pattern A of a:
//  * a in [1, 6]: the step is half the value's leading power of two, so the magnitude index of
//    the lower neighbour is 2 * (biased exponent) + (top mantissa bit) - 252 and 2^32 f is the
//    remaining 22 mantissa bits, A << 10;
//  * a in [1/2, 1): lower neighbour 1/2 (index 1; the formula above gives 0 or 1 there, hence
//    the max), step 1/2, 2^32 f = the 23 mantissa bits, A << 9;
//  * a < 1/2: lower neighbour 0, f = 2 a, and r < 2^33 a is r < ceil(2^33 a) (exact products).
__device__ __forceinline__ uint32_t e2m1_stochastic(float a, uint32_t r)
{
    a = fminf(a, 6.0f);
    const uint32_t A = __float_as_uint(a);
    const bool ge1 = A >= 0x3F800000u, ge_half = A >= 0x3F000000u;
    const uint32_t t_small = (uint32_t)ceilf(a * 8589934592.0f);
    const uint32_t lo = ge_half ? max((A >> 22) - 252u, 1u) : 0u;
    const uint32_t t = ge_half ? A << (ge1 ? 10u : 9u) : t_small;
    return lo + (r < t ? 1u : 0u);
}


// ---------------------------------------------------------------------------- Philox4x32-10 --
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11): ten rounds;
// each multiplies words 0 and 2 by fixed odd constants, swaps the halves of the products in and
// mixes in the other words and the round key; the key advances by fixed Weyl increments.
struct Philox4 {
    uint32_t w[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t p = (uint64_t)0xD2511F53u * c0;
        const uint64_t q = (uint64_t)0xCD9E8D57u * c2;
        // three-input XORs (truth table 0x96) in one gfx950 bitop3 instruction each
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(q >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p >> 32), c3, k1, 0x96);
        c1 = (uint32_t)q;
        c3 = (uint32_t)p;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Philox4 r;
    r.w[0] = c0;
    r.w[1] = c1;
    r.w[2] = c2;
    r.w[3] = c3;
    return r;
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
// Stochastic codes of 8 consecutive values y[0..7] (not yet scaled) whose first element has
// position index0 (a multiple of 8) in the quantized output: two Philox blocks, word k of
// block (index0 / 4 + b) for element 4 b + k.
__device__ __forceinline__ uint32_t encode8_stochastic(const float *y, uint32_t s, uint64_t index0,
                                                       uint32_t key0, uint32_t key1, uint32_t stream_id)
{
    const float mul = e8m0_reciprocal(s);
    const uint64_t c = index0 >> 2;
    const Philox4 r0 = philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), stream_id, 0u, key0, key1);
    const uint64_t c1 = c + 1;
    const Philox4 r1 = philox4x32_10((uint32_t)c1, (uint32_t)(c1 >> 32), stream_id, 0u, key0, key1);
    uint32_t word = 0u, signs = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t rnd = e < 4 ? r0.w[e] : r1.w[e - 4];
        word |= e2m1_stochastic(fabsf(y[e] * mul), rnd) << (4 * e);
        // sign bit of y[e] to bit 4 e + 3 (the sign of the rotated value, also for zeros)
        signs |= (__float_as_uint(y[e]) >> (28 - 4 * e)) & (8u << (4 * e));
    }
    return word | signs;
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

// quant_lane.hpp -- the per-lane steps of the 4-bit quantizers on gfx950: INT4 (shared by
// the activation kernel and the GEMM epilogue that quantizes the next layer's input) and
// NVFP4 (shared by the activation kernel and the weight quantizer).  A lane holds 32
// consecutive channels of one row (one half of a 64-channel group): the lane of one FP6
// MFMA fragment of packed_layout.hpp.  The quantizers are defined as sequences of
// individually rounded fp32 operations (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
// Diffusers", 技术细节 1 step 3 and 技术细节 3): INT4 s = absmax / 7, q = rne(x_hat / s).
#pragma once

#include <stdint.h>

namespace svdq {
namespace lane {

constexpr float kMinNormal = 1.17549435e-38f;

typedef float f32x16v __attribute__((ext_vector_type(16)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// The lane's 32 values in the order of the FP6 conversion: ev[i] is channel 2i (the low
// bf16 of word i), od[i] channel 2i + 1 (the high bf16).
struct Vals {
    f32x16v ev, od;
};

// 32 floats -> 32 FP6 E2M3 fields (value / scale, field 2i from ev[i], 2i+1 from od[i]) in
// six dwords, one v_cvt_scalef32_2xpk16_fp6_f32.  Written as asm with an early-clobber
// result: the instruction reads its 32 source registers over several cycles, so its six
// result registers must not overlap them (left to itself the compiler may place them there).
__device__ __forceinline__ u32x6 cvt_fp6x32(const f32x16v& ev, const f32x16v& od, float scale) {
    u32x6 r;
    asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, %3"
                 : "=&v"(r) : "v"(ev), "v"(od), "v"(scale));
    return r;
}

__device__ __forceinline__ float absmax32(const Vals& v) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fmaxf(fabsf(v.ev[i]), fabsf(v.od[i])));
    return a;
}

// rne(xh / s) for the lane's 32 values, in place, with the fp32 quotient correctly rounded
// as the code's definition requires.  The quotient is estimated as xh * (1/s) (within 2^-22
// relative of the correctly rounded one, i.e. < 2e-6 for |q| <= 8); only when an estimate
// lies within 4e-6 of a half-integer can the correctly rounded quotient round differently,
// and then the lane redoes all 32 with the exact division (smooth32 recomputes x_hat).
// s = absmax / 7 bounds |xh / s| by 7 (up to rounding), so rne never leaves [-7, 7] and the
// definition's clamp to [-8, 7] is the identity.  Codes come out as floats with +0 for 0.
// s = 0 (an all-zero group) gives codes 0.
__device__ __forceinline__ float rne_keep_d(f32x16v& v, int i, float rcp, float dmax) {
#pragma clang fp contract(off)
    const float y = v[i] * rcp;
    const float d = y - __builtin_rintf(y);
    v[i] = y - d;   // = rne(y) exactly, with +0 where it is zero
    return fmaxf(dmax, fabsf(d));
}

// rne(xh / s) for the lane's 32 values in place (see rne_keep_d): `recompute` refills v with
// the smoothed values when the exact division is needed.
template <class Recompute>
__device__ __forceinline__ void int4_codes32_exact(Vals& v, float s, Recompute&& recompute) {
#pragma clang fp contract(off)
    const bool zero = s == 0.0f;
    const float rcp = zero ? 0.0f : 1.0f / s;
    float dmax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        dmax = rne_keep_d(v.ev, i, rcp, dmax);
        dmax = rne_keep_d(v.od, i, rcp, dmax);
    }
    if (!zero && (dmax > 0.499996f || s < kMinNormal)) {
        recompute();
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            v.ev[i] = __builtin_rintf(v.ev[i] / s) + 0.0f;
            v.od[i] = __builtin_rintf(v.od[i] / s) + 0.0f;
        }
    }
}

// Nearest E4M3 ("FN": bias 7, max 448) to v >= 0, ties to even, saturating.
__device__ __forceinline__ uint32_t e4m3_encode(float v) {
    if (!(v > 0.0f)) return 0u;
    if (v >= 448.0f) return 0x7Eu;
    uint32_t u = __float_as_uint(v);
    int e = (int)(u >> 23) - 127;
    if (e < -6) return (uint32_t)__builtin_rintf(v * 512.0f);   // subnormal, 2^-9 steps
    u = u + 0x7FFFFu + ((u >> 20) & 1u);                          // round to 3 mantissa bits
    u &= 0xFFF00000u;
    int er = (int)(u >> 23) - 127;
    return ((uint32_t)(er + 7) << 3) | ((u >> 20) & 7u);
}

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0u) return (float)m * 0.001953125f;
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// NVFP4 for the lane's 32 values: two blocks of 16 (channels 0-15 are ev/od 0-7), each with
// the E4M3 scale sb = e4m3(absmax / (6 S)) and E2M1 codes of v / (e4m3_decode(sb) S) (all
// zero where sb is 0).  d: the 16 code bytes, low nibble the even channel; sbs: the two
// scale bytes (block 0 in the low byte).
//
// The quotient is the correctly rounded fp32 v / dq without a division per value: with
// r = 1 / dq correctly rounded, q0 = v r lies within one ulp of v / dq, so the remainder
// v - q0 dq is exact (one fma) and q0 + remainder * r rounds to v / dq (Markstein's
// theorem on division by a correctly rounded reciprocal).  That needs no overflow and no
// underflow of the remainder: blocks with dq below 2^-100 or quotients that could reach
// 2^100 take the plain division instead.  A quotient that underflows has code 0 whichever
// way it rounds.  The sign of the code is v's (also for v = -0).  The E2M1 rounding is
// v_cvt_scalef32_pk_fp4_f32's with scale 1: nearest, ties to the even code, saturating
// at 6; the first source goes to the low nibble.
__device__ __forceinline__ void nvfp4_codes32(const Vals& v, float S, uint32_t (&d)[4], uint32_t& sbs) {
    const float den = 6.0f * S;
    sbs = 0u;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float a = 0.0f;
#pragma unroll
        for (int i = 8 * b; i < 8 * b + 8; ++i) a = fmaxf(a, fmaxf(fabsf(v.ev[i]), fabsf(v.od[i])));
        const uint32_t sb = e4m3_encode(a / den);
        sbs |= sb << (8 * b);
        const float dq = e4m3_decode(sb) * S;
        const float r = 1.0f / dq;
        float qe[8], qo[8];
        if (sb == 0u || (dq >= 0x1p-100f && a * r < 0x1p100f)) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e0 = v.ev[8 * b + i] * r, o0 = v.od[8 * b + i] * r;
                qe[i] = __builtin_fmaf(__builtin_fmaf(-e0, dq, v.ev[8 * b + i]), r, e0);
                qo[i] = __builtin_fmaf(__builtin_fmaf(-o0, dq, v.od[8 * b + i]), r, o0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qe[i] = v.ev[8 * b + i] / dq;
                qo[i] = v.od[8 * b + i] / dq;
            }
        }
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e = __builtin_copysignf(qe[i], v.ev[8 * b + i]);
            const float o = __builtin_copysignf(qo[i], v.od[8 * b + i]);
            uint32_t& wk = w[i >> 2];
            switch (i & 3) {   // the byte selector must be a constant
                case 0: wk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wk, e, o, 1.0f, 0); break;
                case 1: wk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wk, e, o, 1.0f, 1); break;
                case 2: wk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wk, e, o, 1.0f, 2); break;
                default: wk = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(wk, e, o, 1.0f, 3); break;
            }
        }
        d[2 * b] = sb ? w[0] : 0u;
        d[2 * b + 1] = sb ? w[1] : 0u;
    }
}

}  // namespace lane
}  // namespace svdq

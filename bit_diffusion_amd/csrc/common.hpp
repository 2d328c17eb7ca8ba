// common.hpp -- device-side helpers shared by the gfx950 kernels of libsvdq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

namespace svdq {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t h16) {
    return __uint_as_float(h16 << 16);
}

// fp32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// The 8 bf16 words of a 16-byte register block as an MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float wave_max_xor(float v, int mask) {
    return fmaxf(v, __shfl_xor(v, mask, kWave));
}

// GELU, tanh form: 0.5 y (1 + tanh(u)), u = sqrt(2/pi) (y + 0.044715 y^3).  Evaluated as
// the identical y / (1 + exp(-2u)), which keeps full relative accuracy for negative y where
// 1 + tanh(u) would cancel, with the hardware's exp2 and reciprocal (about 1 ulp each):
// e = 2^(-2 log2(e) u) and y * rcp(1 + e).  A relative error d in e moves the result by
// at most e / (1 + e)^2 * d <= d / 4 of y, so the argument's rounding (|d| up to |x| ulp
// for x = -2 log2(e) u) is damped where |x| is large; the result is within a few ulp of
// |y|.  e overflows to inf for large negative y, whose reciprocal 0 gives the limit -0.
__device__ __forceinline__ float gelu_tanh(float y) {
    const float c = 0.7978845608028654f;   // sqrt(2 / pi)
    const float u = c * (y + 0.044715f * y * y * y);
    const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * u);   // -2 log2(e) u
    return y * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace svdq

// quant.hip -- activation kernels of the SVDQ W4A4 linear on gfx950.
//
// One pass over the bf16 activations X does three things
// (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 1,
//  "SVDQuant 的核心思路" steps 1, 3 and 4):
//   * smoothing: x_hat = fp32(x) * smooth_inv[k]  (outliers migrated into the weights);
//   * 4-bit quantization of x_hat with per-group scales, codes packed two per byte;
//   * the low-rank down-projection lora_act = X . L1^T on the same registers (bf16 MFMA),
//     so the 16-bit branch costs no extra pass over X.
//
// Work mapping: a block owns 16 token rows; each of its 8 waves walks a strided subset of
// the 64-channel groups.  Lane l holds row (l % 16) and the 16 consecutive channels
// 16 * (l / 16) .. +15 of the current group, i.e. a 16x64 tile per wave and step, which is
// also the A-operand layout of two v_mfma_f32_16x16x32_bf16 (one per 32-channel half).
// The group absmax is a max over the four lanes of a row (xor-shuffles 16, 32).
#include "common.hpp"
#include "launch.hpp"

// The quantizer is defined as a sequence of individually rounded fp32 operations.
#pragma clang fp contract(off)

namespace svdq {
namespace {

constexpr int kRows = 16;
constexpr int kWaves = 8;
constexpr float kMinNormal = 1.17549435e-38f;

// rne(xh / s) clamped to [-8, 7], with the fp32 quotient correctly rounded as the code's
// definition requires.  The quotient is first estimated as xh * (1/s) (relative error
// below 2^-23, i.e. < 1e-6 for |q| <= 8); only when that estimate lies within 4e-6 of a
// half-integer can the correctly rounded quotient round differently, and then the exact
// division decides.
__device__ __forceinline__ int int4_code(float xh, float s, float rcp, bool exact_only) {
    float y = xh * rcp;
    float r = __builtin_rintf(y);
    if (exact_only || fabsf(fabsf(y - r) - 0.5f) < 4.0e-6f) r = __builtin_rintf(xh / s);
    r = fminf(fmaxf(r, -8.0f), 7.0f);
    return (int)r;
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

// Nearest E2M1 magnitude (0, .5, 1, 1.5, 2, 3, 4, 6), ties to the even code, saturating;
// sign in bit 3.
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    float a = fabsf(v);
    uint32_t c = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
               : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
    return c | ((__float_as_uint(v) >> 28) & 8u);
}

struct Tile16 {
    uint4 xv0, xv1;      // 16 bf16 of one row
    float xh[16];        // smoothed fp32
};

__device__ __forceinline__ void load_tile(Tile16& t, const uint16_t* xr, const float* si, int k0) {
    t.xv0 = *reinterpret_cast<const uint4*>(xr + k0);
    t.xv1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
    const float4* sp = reinterpret_cast<const float4*>(si + k0);
    float4 s[4] = {sp[0], sp[1], sp[2], sp[3]};
    uint32_t w[8] = {t.xv0.x, t.xv0.y, t.xv0.z, t.xv0.w, t.xv1.x, t.xv1.y, t.xv1.z, t.xv1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        float sv = (&s[i >> 2].x)[i & 3];
        t.xh[i] = bf16_to_f32(h) * sv;
    }
}

// Accumulate the 16x(16*RB) block of X . L1^T for this 64-channel group.
template <int RB>
__device__ __forceinline__ void lowrank_step(f32x4 (&acc)[RB > 0 ? RB : 1], const Tile16& t,
                                             const uint16_t* l1, int K, int rl, int k0) {
    if constexpr (RB > 0) {
        bf16x8 a0 = as_bf16x8(t.xv0), a1 = as_bf16x8(t.xv1);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const uint16_t* lr = l1 + (int64_t)(b * 16 + rl) * K + k0;
            uint4 b0 = *reinterpret_cast<const uint4*>(lr);
            uint4 b1 = *reinterpret_cast<const uint4*>(lr + 8);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(b0), acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(b1), acc[b], 0, 0, 0);
        }
    }
}

// Sum the per-wave partial products over the waves (fixed order) and store bf16 lora_act.
template <int RB>
__device__ __forceinline__ void lowrank_finish(f32x4 (&acc)[RB > 0 ? RB : 1], float* red,
                                               int64_t m0, int64_t M, uint16_t* lora) {
    if constexpr (RB > 0) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red[((wave * RB + b) * 16 + (4 * (lane >> 4) + i)) * 16 + (lane & 15)] = acc[b][i];
        __syncthreads();
        for (int t = threadIdx.x; t < 256 * RB; t += blockDim.x) {
            int b = t >> 8, rr = (t >> 4) & 15, cc = t & 15;
            float s = 0.0f;
            for (int w = 0; w < kWaves; ++w) s += red[((w * RB + b) * 16 + rr) * 16 + cc];
            int64_t m = m0 + rr;
            if (m < M) lora[m * (RB * 16) + b * 16 + cc] = (uint16_t)f32_to_bf16(s);
        }
    }
}

template <int RB>
__global__ __launch_bounds__(kWaves * 64) void quant_act_int4_kernel(
    int64_t M, int K, const uint16_t* __restrict__ x, const float* __restrict__ smooth_inv,
    const uint16_t* __restrict__ l1, uint8_t* __restrict__ codes, float* __restrict__ scales,
    uint16_t* __restrict__ lora) {
    __shared__ float red[RB > 0 ? kWaves * 256 * RB : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * kRows;
    const int rl = lane & 15, kc = (lane >> 4) * 16;
    const int64_t row = m0 + rl;
    const bool valid = row < M;
    const uint16_t* xr = x + (valid ? row : M - 1) * (int64_t)K;
    const int G = K >> 6;
    f32x4 acc[RB > 0 ? RB : 1];
#pragma unroll
    for (int b = 0; b < (RB > 0 ? RB : 1); ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g = wave; g < G; g += kWaves) {
        const int k0 = g * 64 + kc;
        Tile16 t;
        load_tile(t, xr, smooth_inv, k0);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(t.xh[i]));
        a = wave_max_xor(a, 16);
        a = wave_max_xor(a, 32);
        const float s = a / 7.0f;
        uint32_t p0 = 0u, p1 = 0u;
        if (s != 0.0f) {
            const float rcp = 1.0f / s;
            const bool exact_only = s < kMinNormal;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t nib = (uint32_t)int4_code(t.xh[i], s, rcp, exact_only) & 15u;
                if (i < 8) p0 |= nib << (4 * i);
                else p1 |= nib << (4 * (i - 8));
            }
        }
        if (valid) {
            *reinterpret_cast<uint2*>(codes + row * (K / 2) + k0 / 2) = make_uint2(p0, p1);
            if (kc == 0) scales[row * G + g] = s;
        }
        lowrank_step<RB>(acc, t, l1, K, rl, k0);
    }
    lowrank_finish<RB>(acc, red, m0, M, lora);
}

template <int RB>
__global__ __launch_bounds__(kWaves * 64) void quant_act_nvfp4_kernel(
    int64_t M, int K, const uint16_t* __restrict__ x, const float* __restrict__ smooth_inv,
    const uint16_t* __restrict__ l1, float S, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, uint16_t* __restrict__ lora) {
    __shared__ float red[RB > 0 ? kWaves * 256 * RB : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * kRows;
    const int rl = lane & 15, kc = (lane >> 4) * 16;
    const int64_t row = m0 + rl;
    const bool valid = row < M;
    const uint16_t* xr = x + (valid ? row : M - 1) * (int64_t)K;
    const int G = K >> 6;
    const float den = 6.0f * S;
    f32x4 acc[RB > 0 ? RB : 1];
#pragma unroll
    for (int b = 0; b < (RB > 0 ? RB : 1); ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int g = wave; g < G; g += kWaves) {
        const int k0 = g * 64 + kc;   // this lane's 16 channels are one NVFP4 block
        Tile16 t;
        load_tile(t, xr, smooth_inv, k0);
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(t.xh[i]));
        const uint32_t sb = e4m3_encode(a / den);
        uint32_t p0 = 0u, p1 = 0u;
        if (sb != 0u) {
            const float d = e4m3_decode(sb) * S;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                uint32_t c = e2m1_encode(t.xh[i] / d);
                if (i < 8) p0 |= c << (4 * i);
                else p1 |= c << (4 * (i - 8));
            }
        }
        if (valid) {
            *reinterpret_cast<uint2*>(codes + row * (K / 2) + k0 / 2) = make_uint2(p0, p1);
            scales[row * (K / 16) + k0 / 16] = (uint8_t)sb;
        }
        lowrank_step<RB>(acc, t, l1, K, rl, k0);
    }
    lowrank_finish<RB>(acc, red, m0, M, lora);
}

template <int RB>
void launch_int4(const QuantArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.M + kRows - 1) / kRows)), block(kWaves * 64);
    hipLaunchKernelGGL(quant_act_int4_kernel<RB>, grid, block, 0, st, a.M, a.K,
                       (const uint16_t*)a.x, a.smooth_inv, (const uint16_t*)a.l1,
                       (uint8_t*)a.codes, (float*)a.scales, (uint16_t*)a.lora);
}

template <int RB>
void launch_nvfp4(const QuantArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.M + kRows - 1) / kRows)), block(kWaves * 64);
    hipLaunchKernelGGL(quant_act_nvfp4_kernel<RB>, grid, block, 0, st, a.M, a.K,
                       (const uint16_t*)a.x, a.smooth_inv, (const uint16_t*)a.l1, a.S,
                       (uint8_t*)a.codes, (uint8_t*)a.scales, (uint16_t*)a.lora);
}

}  // namespace

void launch_quantize_act(const QuantArgs& a, hipStream_t st) {
    const int rb = a.r / 16;
    if (a.nvfp4) {
        switch (rb) {
            case 0: launch_nvfp4<0>(a, st); break;
            case 1: launch_nvfp4<1>(a, st); break;
            case 2: launch_nvfp4<2>(a, st); break;
            case 3: launch_nvfp4<3>(a, st); break;
            case 4: launch_nvfp4<4>(a, st); break;
            case 5: launch_nvfp4<5>(a, st); break;
            case 6: launch_nvfp4<6>(a, st); break;
            case 7: launch_nvfp4<7>(a, st); break;
            default: launch_nvfp4<8>(a, st); break;
        }
    } else {
        switch (rb) {
            case 0: launch_int4<0>(a, st); break;
            case 1: launch_int4<1>(a, st); break;
            case 2: launch_int4<2>(a, st); break;
            case 3: launch_int4<3>(a, st); break;
            case 4: launch_int4<4>(a, st); break;
            case 5: launch_int4<5>(a, st); break;
            case 6: launch_int4<6>(a, st); break;
            case 7: launch_int4<7>(a, st); break;
            default: launch_int4<8>(a, st); break;
        }
    }
}

}  // namespace svdq

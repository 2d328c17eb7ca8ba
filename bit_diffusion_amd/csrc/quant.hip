// quant.hip -- activation kernels of the SVDQ W4A4 linear on gfx950.
//
// One pass over the bf16 activations X does three things
// (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 1,
//  "SVDQuant 的核心思路" steps 1, 3 and 4):
//   * smoothing: x_hat = fp32(x) * smooth_inv[k]  (outliers migrated into the weights);
//   * 4-bit quantization of x_hat with per-group scales, written either as two's-complement
//     nibbles (two per byte) or directly as the MFMA-ready FP6 fragments of
//     packed_layout.hpp that the fast GEMM consumes;
//   * the low-rank down-projection lora_act = X . L1^T on the same registers (bf16 MFMA),
//     so the 16-bit branch costs no extra pass over X.
//
// Work mapping: a block of 16 waves owns 16 token rows; wave w walks groups w, w+16, ...
// Lane l holds row (l % 16) and the 16 consecutive channels 16 * (l / 16) .. +15 of the
// current 64-channel group: the A-operand layout of two v_mfma_f32_16x16x32_bf16 (one per
// 32-channel half) for the low-rank down-projection.  The group absmax is a max over the
// four lanes of a row (xor-shuffles 16, 32).  Each wave keeps the loads of its next few
// groups in flight while it processes the current one; smooth_inv sits in LDS.
#include "common.hpp"
#include "launch.hpp"
#include "packed_layout.hpp"

// The quantizer is defined as a sequence of individually rounded fp32 operations.
#pragma clang fp contract(off)

namespace svdq {
namespace {

constexpr int kRows = 16;
constexpr float kMinNormal = 1.17549435e-38f;
constexpr int kQWaves = 16;
constexpr size_t kQuantMaxLds = 160 * 1024;
constexpr int kQThreads = kQWaves * 64;

enum Mode { kInt4Nibbles = 0, kInt4Packed = 1, kNvfp4Nibbles = 2 };

// Up to rank 32 the L1 slices travel with the activations, and two (rank 32) or three
// (rank <= 16) groups per wave are in flight; beyond that the registers would spill, so one
// group is in flight and L1 is loaded when it is used.
template <int RB>
constexpr bool kPrefetchL1 = RB <= 2;
template <int RB>
constexpr int kAhead = RB <= 1 ? 3 : RB == 2 ? 2 : 1;

template <int RB>
struct Stage16 {
    uint4 xv0, xv1;                                    // 16 bf16 of one row
    uint4 l1v[kPrefetchL1<RB> && RB > 0 ? 2 * RB : 1]; // L1 rows (16 b + row), this group
};

template <int RB>
__device__ __forceinline__ void load_stage(Stage16<RB>& st, const uint16_t* xr, const uint16_t* l1,
                                           int K, int rl, int k0) {
    st.xv0 = *reinterpret_cast<const uint4*>(xr + k0);
    st.xv1 = *reinterpret_cast<const uint4*>(xr + k0 + 8);
    if constexpr (kPrefetchL1<RB>)
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const uint16_t* lr = l1 + (int64_t)(b * 16 + rl) * K + k0;
        st.l1v[2 * b] = *reinterpret_cast<const uint4*>(lr);
        st.l1v[2 * b + 1] = *reinterpret_cast<const uint4*>(lr + 8);
    }
}

// x_hat = fp32(x) * smooth_inv for the lane's 16 channels (smooth_inv from LDS); rows
// beyond M read as zero.
template <int RB>
__device__ __forceinline__ void smooth16(float (&xh)[16], const Stage16<RB>& st, const float* si,
                                         bool valid) {
    const float4* sp = reinterpret_cast<const float4*>(si);
    const float4 s4[4] = {sp[0], sp[1], sp[2], sp[3]};
    const uint32_t w[8] = {st.xv0.x, st.xv0.y, st.xv0.z, st.xv0.w,
                           st.xv1.x, st.xv1.y, st.xv1.z, st.xv1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t h = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
        xh[i] = valid ? bf16_to_f32(h) * (&s4[i >> 2].x)[i & 3] : 0.0f;
    }
}

// rne(xh / s) clamped to [-8, 7] for the lane's 16 values, with the fp32 quotient
// correctly rounded as the code's definition requires.  The quotient is estimated as
// xh * (1/s) (within 2^-22 relative of the correctly rounded one, i.e. < 2e-6 for
// |q| <= 8); only when an estimate lies within 4e-6 of a half-integer can the correctly
// rounded quotient round differently, and then the lane redoes all 16 with the exact
// division.  s = 0 (an all-zero group) gives codes 0.
__device__ __forceinline__ void int4_codes(const float (&xh)[16], float s, float (&q)[16]) {
    const bool zero = s == 0.0f;
    const float rcp = zero ? 0.0f : 1.0f / s;
    bool redo = s < kMinNormal && !zero;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float y = xh[i] * rcp;
        q[i] = __builtin_rintf(y);
        redo |= fabsf(y - q[i]) > 0.499996f;
    }
    if (redo && !zero) {
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = __builtin_rintf(xh[i] / s);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = fminf(fmaxf(q[i], -8.0f), 7.0f);
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

template <int RB>
__device__ __forceinline__ void lowrank_mfma(f32x4 (&acc)[RB > 0 ? RB : 1], const Stage16<RB>& st,
                                             const uint16_t* l1, int K, int rl, int k0) {
    if constexpr (RB > 0) {
        const bf16x8 a0 = as_bf16x8(st.xv0), a1 = as_bf16x8(st.xv1);
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            uint4 v0, v1;
            if constexpr (kPrefetchL1<RB>) {
                v0 = st.l1v[2 * b];
                v1 = st.l1v[2 * b + 1];
            } else {
                const uint16_t* lr = l1 + (int64_t)(b * 16 + rl) * K + k0;
                v0 = *reinterpret_cast<const uint4*>(lr);
                v1 = *reinterpret_cast<const uint4*>(lr + 8);
            }
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, as_bf16x8(v0), acc[b], 0, 0, 0);
            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, as_bf16x8(v1), acc[b], 0, 0, 0);
        }
    }
}

// Sum the 16 waves' partial low-rank products in a fixed tree order and store bf16 lora_act.
// red holds 8 waves x RB x 256 floats.
template <int RB>
__device__ __forceinline__ void lowrank_finish(f32x4 (&acc)[RB > 0 ? RB : 1], float* red,
                                               int64_t m0, int64_t M, uint16_t* lora) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if constexpr (RB > 0) {
#pragma unroll
        for (int half = kQWaves / 2; half >= 1; half >>= 1) {
            if (wave >= half && wave < 2 * half) {
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    *reinterpret_cast<f32x4*>(&red[(((wave - half) * RB + b) * 64 + lane) * 4]) = acc[b];
            }
            __syncthreads();
            if (wave < half) {
#pragma unroll
                for (int b = 0; b < RB; ++b)
                    acc[b] += *reinterpret_cast<const f32x4*>(&red[((wave * RB + b) * 64 + lane) * 4]);
            }
            __syncthreads();
        }
        if (wave == 0) {
            // 16x16 output layout: lane holds rows 4 * (lane / 16) + i, column lane % 16
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t m = m0 + 4 * (lane >> 4) + i;
                    if (m < M) lora[m * (RB * 16) + b * 16 + (lane & 15)] = (uint16_t)f32_to_bf16(acc[b][i]);
                }
        }
    }
}

// Quantize one (16 rows x 64 channels) group held by the wave and write its codes.
template <int MODE>
__device__ __forceinline__ void quantize_group(const float (&xh)[16], int64_t row, bool valid,
                                               int g, int G, int K, int kc, float den,
                                               const QuantArgs& p) {
    const int quarter = kc >> 4;
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(xh[i]));
    if constexpr (MODE != kNvfp4Nibbles) {
        // INT4: the 64-channel group spans the four lanes of this row
        a = wave_max_xor(a, 16);
        a = wave_max_xor(a, 32);
        const float s = a / 7.0f;
        float q[16];
        int4_codes(xh, s, q);
        if constexpr (MODE == kInt4Nibbles) {
            uint32_t p0 = 0u, p1 = 0u;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t nib = (uint32_t)(int)q[i] & 15u;
                if (i < 8) p0 |= nib << (4 * i);
                else p1 |= nib << (4 * (i - 8));
            }
            if (valid) {
                *reinterpret_cast<uint2*>((uint8_t*)p.codes + row * (K / 2) + (g * 64 + kc) / 2) =
                    make_uint2(p0, p1);
                if (quarter == 0) reinterpret_cast<float*>(p.scales)[row * G + g] = s;
            }
        } else {
            // FP6 fields (sign << 5 | |q|) of channels 16 (quarter & 1) + i of MFMA lane
            // L = row % 32 + 32 (quarter >> 1): bits 96 (quarter & 1) + 6 i of its six dwords
            uint32_t d[3] = {0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qi = (int)q[i];
                const uint32_t f = (uint32_t)fabsf(q[i]) | (((uint32_t)qi >> 26) & 32u);
                const int pos = 6 * i;
                d[pos >> 5] |= f << (pos & 31);
                if ((pos & 31) > 26) d[(pos >> 5) + 1] |= f >> (32 - (pos & 31));
            }
            const int r32 = (int)(row & 31), L = r32 + 32 * (quarter >> 1);
            uint8_t* blk = (uint8_t*)p.codes + packed::act_block(row, g, G);
            const bool odd = quarter & 1;
            // even quarter: dwords 0-2 of the lane; odd quarter: dwords 3-5
            *reinterpret_cast<uint2*>(blk + (odd ? packed::frag_dword(L, 4) : packed::frag_dword(L, 0))) =
                odd ? make_uint2(d[1], d[2]) : make_uint2(d[0], d[1]);
            *reinterpret_cast<uint32_t*>(blk + (odd ? packed::frag_dword(L, 3) : packed::frag_dword(L, 2))) =
                odd ? d[0] : d[2];
            if (quarter == 0) {
                const uint32_t hi = f32_to_bf16(s);
                const uint32_t lo = f32_to_bf16(s - __uint_as_float(hi << 16));
                *reinterpret_cast<uint32_t*>(blk + packed::kFrag + 4 * r32) = hi | (lo << 16);
                if (valid && p.scales) reinterpret_cast<float*>(p.scales)[row * G + g] = s;
            }
        }
    } else {
        // NVFP4: this lane's 16 channels are one block
        const uint32_t sb = e4m3_encode(a / den);
        uint32_t p0 = 0u, p1 = 0u;
        if (sb != 0u) {
            const float dq = e4m3_decode(sb) * p.S;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t c = e2m1_encode(xh[i] / dq);
                if (i < 8) p0 |= c << (4 * i);
                else p1 |= c << (4 * (i - 8));
            }
        }
        if (valid) {
            const int k0 = g * 64 + kc;
            reinterpret_cast<uint8_t*>(p.scales)[row * (K / 16) + k0 / 16] = (uint8_t)sb;
            *reinterpret_cast<uint2*>((uint8_t*)p.codes + row * (K / 2) + k0 / 2) = make_uint2(p0, p1);
        }
    }
}

template <int RB, int MODE>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(QuantArgs p) {
    extern __shared__ __align__(16) float qsm[];
    const int K = p.K;
    const int64_t M = p.M;
    float* si_lds = qsm;                     // K floats
    float* red = qsm + K;                    // 8 * RB * 256 floats
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.x * kRows;
    const int rl = lane & 15, kc = (lane >> 4) * 16;
    const int64_t row = m0 + rl;
    const bool valid = row < M;
    const uint16_t* x = (const uint16_t*)p.x;
    const uint16_t* l1 = (const uint16_t*)p.l1;
    const uint16_t* xr = x + (valid ? row : M - 1) * (int64_t)K;
    const int G = K >> 6;
    const int ng = G > wave ? (G - wave + kQWaves - 1) / kQWaves : 0;   // this wave's groups
    constexpr int NA = kAhead<RB>;
    f32x4 acc[RB > 0 ? RB : 1];
#pragma unroll
    for (int b = 0; b < (RB > 0 ? RB : 1); ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stage16<RB> st[NA];
#pragma unroll
    for (int s = 0; s < NA; ++s)
        if (s < ng) load_stage<RB>(st[s], xr, l1, K, rl, (wave + s * kQWaves) * 64 + kc);
    for (int i = threadIdx.x * 4; i < K; i += kQThreads * 4)
        *reinterpret_cast<float4*>(si_lds + i) = *reinterpret_cast<const float4*>(p.smooth_inv + i);
    __syncthreads();
    const float den = 6.0f * p.S;

    for (int it0 = 0; it0 < ng; it0 += NA) {
#pragma unroll
        for (int s = 0; s < NA; ++s) {
            const int it = it0 + s;
            if (it < ng) {
                const int g = wave + it * kQWaves;
                const int k0 = g * 64 + kc;
                float xh[16];
                smooth16<RB>(xh, st[s], si_lds + k0, valid);
                quantize_group<MODE>(xh, row, valid, g, G, K, kc, den, p);
                lowrank_mfma<RB>(acc, st[s], l1, K, rl, k0);
                if (it + NA < ng) load_stage<RB>(st[s], xr, l1, K, rl, k0 + NA * kQWaves * 64);
            }
        }
    }
    lowrank_finish<RB>(acc, red, m0, M, (uint16_t*)p.lora);
}

template <int RB, int MODE>
void launch_mode(const QuantArgs& a, int64_t rows, hipStream_t st) {
    const size_t lds = ((size_t)a.K + 8 * (size_t)RB * 256) * sizeof(float);
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)quant_act_kernel<RB, MODE>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kQuantMaxLds);
        attr_set = true;
    }
    hipLaunchKernelGGL((quant_act_kernel<RB, MODE>), dim3((unsigned)((rows + kRows - 1) / kRows)),
                       dim3(kQThreads), lds, st, a);
}

template <int RB>
void launch_rb(const QuantArgs& a, hipStream_t st) {
    if (a.mode == kInt4Packed) {
        // cover the padded rows of the packed layout so they hold zero codes and scales
        const int64_t rows = (a.M + packed::kBM - 1) / packed::kBM * packed::kBM;
        launch_mode<RB, kInt4Packed>(a, rows, st);
    } else if (a.mode == kNvfp4Nibbles) {
        launch_mode<RB, kNvfp4Nibbles>(a, a.M, st);
    } else {
        launch_mode<RB, kInt4Nibbles>(a, a.M, st);
    }
}

}  // namespace

size_t quantize_act_lds_bytes(int K, int r) {
    return ((size_t)K + 8 * (size_t)(r / 16) * 256) * sizeof(float);
}

void launch_quantize_act(const QuantArgs& a, hipStream_t st) {
    switch (a.r / 16) {
        case 0: launch_rb<0>(a, st); break;
        case 1: launch_rb<1>(a, st); break;
        case 2: launch_rb<2>(a, st); break;
        case 3: launch_rb<3>(a, st); break;
        case 4: launch_rb<4>(a, st); break;
        case 5: launch_rb<5>(a, st); break;
        case 6: launch_rb<6>(a, st); break;
        case 7: launch_rb<7>(a, st); break;
        default: launch_rb<8>(a, st); break;
    }
}

}  // namespace svdq

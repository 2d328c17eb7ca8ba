// gemm_nvfp4.hip -- NVFP4 variant of the W4A4 GEMM (page "Hugging Face 把 Nunchaku 4-bit
// Diffusion 接到 Diffusers", 技术细节 3: svdq_w4a4 with precision nvfp4), with the same
// low-rank / bias / GELU epilogue as the INT4 kernel.
//
//   y[m,n] = S_a S_w sum_k (e_a[m,k] sb_a[m,k/16]) (e_w[n,k] sb_w[n,k/16]) + lowrank + b
//
// gfx950's scaled MFMA takes power-of-two (E8M0) block scales on 32-element blocks, which
// cannot carry NVFP4's E4M3 scales on 16-element blocks.  Instead each E2M1 value (at
// most 2 significant bits) is multiplied by its E4M3 block scale (at most 4 significant
// bits): the product has at most 6 significant bits and a small exponent range, so it is
// exact in bf16.  The tile is dequantized once per block into LDS and contracted with
// v_mfma_f32_32x32x16_bf16 in fp32; S_a * S_w is applied once in the epilogue.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

constexpr int BM = 128, BN = 128, BK = 64, kThreads = 256;
constexpr int kLdsRow = BK + 8;   // bf16 elements per LDS row (16-byte pad)

struct Smem {
    uint16_t a[BM * kLdsRow];
    uint16_t b[BN * kLdsRow];
};

__device__ __forceinline__ float e2m1_value(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    float mag = e ? __uint_as_float(((e + 126u) << 23) | (m << 22)) : (m ? 0.5f : 0.0f);
    return (c & 8u) ? -mag : mag;
}

__device__ __forceinline__ float e4m3_value(uint32_t b) {
    uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 0u) return (float)m * 0.001953125f;
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// 32 codes (16 bytes) + their two block scales -> 32 exact bf16 values in LDS.
__device__ __forceinline__ void dequant32(uint4 c, uint32_t sc2, uint16_t* dst) {
    const float s0 = e4m3_value(sc2 & 0xFFu), s1 = e4m3_value((sc2 >> 8) & 0xFFu);
    uint32_t w[4] = {c.x, c.y, c.z, c.w};
    uint32_t outw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t byte = (w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
        const float s = i < 8 ? s0 : s1;
        const uint32_t lo = __float_as_uint(e2m1_value(byte & 0xFu) * s) >> 16;
        const uint32_t hi = __float_as_uint(e2m1_value(byte >> 4) * s) >> 16;
        outw[i] = lo | (hi << 16);
    }
    uint4* d = reinterpret_cast<uint4*>(dst);
#pragma unroll
    for (int i = 0; i < 4; ++i) d[i] = make_uint4(outw[4 * i], outw[4 * i + 1], outw[4 * i + 2], outw[4 * i + 3]);
}

__global__ __launch_bounds__(kThreads) void gemm_nvfp4_v0_kernel(GemmArgs p) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, K = p.K;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const uint8_t* wcodes = (const uint8_t*)p.wcodes;
    const uint8_t* ascales = (const uint8_t*)p.ascales;
    const uint8_t* wscales = (const uint8_t*)p.wscales;

    const int lrow = tid >> 1, lhalf = tid & 1;
    const int64_t am = (m0 + lrow < M) ? m0 + lrow : M - 1;
    const int64_t bn = (n0 + lrow < N) ? n0 + lrow : N - 1;
    const uint8_t* ag = acodes + am * (K / 2) + lhalf * 16;
    const uint8_t* bg = wcodes + bn * (K / 2) + lhalf * 16;
    const uint8_t* asg = ascales + am * (K / 16) + lhalf * 2;
    const uint8_t* bsg = wscales + bn * (K / 16) + lhalf * 2;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int fr = lane & 31, fh = lane >> 5;
    for (int k0 = 0; k0 < K; k0 += BK) {
        const uint4 ca = *reinterpret_cast<const uint4*>(ag + k0 / 2);
        const uint4 cb = *reinterpret_cast<const uint4*>(bg + k0 / 2);
        const uint32_t sa2 = asg[k0 / 16] | ((uint32_t)asg[k0 / 16 + 1] << 8);
        const uint32_t sb2 = bsg[k0 / 16] | ((uint32_t)bsg[k0 / 16 + 1] << 8);
        __syncthreads();   // previous step's readers are done with the tile
        dequant32(ca, sa2, &sm.a[lrow * kLdsRow + lhalf * 32]);
        dequant32(cb, sb2, &sm.b[lrow * kLdsRow + lhalf * 32]);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 va[2], vb[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                va[f] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &sm.a[(wm * 64 + f * 32 + fr) * kLdsRow + kk + 8 * fh]));
                vb[f] = as_bf16x8(*reinterpret_cast<const uint4*>(
                    &sm.b[(wn * 64 + f * 32 + fr) * kLdsRow + kk + 8 * fh]));
            }
#pragma unroll
            for (int fa = 0; fa < 2; ++fa)
#pragma unroll
                for (int fb = 0; fb < 2; ++fb)
                    acc[fa][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[fa], vb[fb],
                                                                          acc[fa][fb], 0, 0, 0);
        }
    }

    const float sasw = p.Sa * p.Sw;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] *= sasw;

    const uint16_t* lora = (const uint16_t*)p.lora;
    const uint16_t* l2 = (const uint16_t*)p.l2;
    const int r = p.r;
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
        int64_t mrow = m0 + wm * 64 + fa * 32 + fr;
        if (mrow >= M) mrow = M - 1;
#pragma unroll
        for (int fb = 0; fb < 2; ++fb) {
            int ncol = n0 + wn * 64 + fb * 32 + fr;
            if (ncol >= N) ncol = N - 1;
            for (int kk = 0; kk < r; kk += 16) {
                uint4 va = *reinterpret_cast<const uint4*>(lora + mrow * r + kk + 8 * fh);
                uint4 vb = *reinterpret_cast<const uint4*>(l2 + (int64_t)ncol * r + kk + 8 * fh);
                acc[fa][fb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(vb),
                                                                      acc[fa][fb], 0, 0, 0);
            }
        }
    }
    const uint16_t* bias = (const uint16_t*)p.bias;
#pragma unroll
    for (int fb = 0; fb < 2; ++fb) {
        const int col = n0 + wn * 64 + fb * 32 + fr;
        const bool cok = col < N;
        const float bv = (bias && cok) ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
        for (int fa = 0; fa < 2; ++fa)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + fa * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                float v = acc[fa][fb][e] + bv;
                if (p.act == 1) v = gelu_tanh(v);
                if (cok && row < M) {
                    if (p.out_bf16)
                        ((uint16_t*)p.out)[row * N + col] = (uint16_t)f32_to_bf16(v);
                    else
                        ((float*)p.out)[row * N + col] = v;
                }
            }
    }
}

}  // namespace

void launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_nvfp4_v0_kernel, grid, dim3(kThreads), 0, st, a);
}

}  // namespace svdq

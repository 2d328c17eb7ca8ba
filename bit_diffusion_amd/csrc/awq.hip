// awq.hip -- AWQ W4A16 GEMV / skinny GEMM for modulation layers (page "Diffusers Natively
// Integrates Nunchaku Lite ...", third paragraph: sensitive or bandwidth-bound modulation
// layers keep 16-bit activations with 4-bit weights; kernel family awq_w4a16, page "Hugging
// Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 3).
//
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] (q[n,k] - z[n,g]) + b[n]
//
// Reference kernel ("v0"): one wave per output row n; each lane streams 16-byte chunks
// (32 codes, half a group) of that row and forms sum_k x*(q - z) for up to 4 token rows at
// a time in fp32, scaled once per half-group; a wave reduction finishes the dot products.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kMB = 4;   // token rows per pass over the weights

__global__ __launch_bounds__(kWavesPerBlock * 64) void awq_gemv_v0_kernel(AwqArgs p) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = blockIdx.x * kWavesPerBlock + wave;
    if (n >= p.N) return;   // whole wave exits together
    const int K = p.K, G = K >> 6, chunks = K >> 5;
    const uint8_t* qrow = (const uint8_t*)p.qweight + (int64_t)n * (K / 2);
    const uint16_t* srow = (const uint16_t*)p.scales + (int64_t)n * G;
    const uint16_t* zrow = (const uint16_t*)p.zeros + (int64_t)n * G;
    const uint16_t* x = (const uint16_t*)p.x;
    const float bv = p.bias ? bf16_to_f32(((const uint16_t*)p.bias)[n]) : 0.0f;

    for (int64_t mc = 0; mc < p.M; mc += kMB) {
        const int mb = (p.M - mc) < kMB ? (int)(p.M - mc) : kMB;
        float acc[kMB] = {0.f, 0.f, 0.f, 0.f};
        for (int c = lane; c < chunks; c += 64) {
            const uint4 qv = *reinterpret_cast<const uint4*>(qrow + c * 16);
            const int g = c >> 1;
            const float sc = bf16_to_f32(srow[g]);
            const float z = bf16_to_f32(zrow[g]);
            float qf[32];
            const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
            for (int i = 0; i < 32; ++i) qf[i] = (float)((w[i >> 3] >> (4 * (i & 7))) & 15u) - z;
#pragma unroll
            for (int mm = 0; mm < kMB; ++mm) {
                if (mm < mb) {
                    const uint4* xp = reinterpret_cast<const uint4*>(x + (mc + mm) * K + c * 32);
                    float s = 0.0f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint4 xv = xp[j];
                        const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            s += bf16_to_f32(xw[t] & 0xFFFFu) * qf[8 * j + 2 * t];
                            s += bf16_to_f32(xw[t] >> 16) * qf[8 * j + 2 * t + 1];
                        }
                    }
                    acc[mm] += s * sc;
                }
            }
        }
#pragma unroll
        for (int mm = 0; mm < kMB; ++mm) {
            float v = acc[mm];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
            if (lane == 0 && mm < mb) {
                v += bv;
                const int64_t idx = (mc + mm) * p.N + n;
                if (p.out_bf16) ((uint16_t*)p.out)[idx] = (uint16_t)f32_to_bf16(v);
                else ((float*)p.out)[idx] = v;
            }
        }
    }
}

}  // namespace

void launch_awq_gemv(const AwqArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + kWavesPerBlock - 1) / kWavesPerBlock));
    hipLaunchKernelGGL(awq_gemv_v0_kernel, grid, dim3(kWavesPerBlock * 64), 0, st, a);
}

}  // namespace svdq

// gemm_int4.hip -- INT4 W4A4 GEMM with the low-rank up-projection, bias and optional
// GELU in its epilogue (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers",
// 技术细节 1 step 4; kernel family svdq_w4a4 / int4, 技术细节 3).
//
//   y[m,n] = sum_g sa[m,g] sw[n,g] D_g[m,n] + sum_j lora[m,j] l2[n,j] + b[n],
//   D_g    = sum_{k in group g} qa[m,k] qw[n,k]   (exact integer, 64 channels per group)
//
// Reference kernel ("v0"): a 128x128 output tile per 256-thread block, 2x2 waves of 64x64.
// Per 64-channel group the packed nibbles of A and W go HBM -> registers -> LDS (double
// buffered, rows padded to 48 bytes so the 16-byte LDS reads of 16 consecutive lanes hit
// distinct banks).  Each wave expands its fragments to int8 in registers as 16*q (a nibble
// masked into the high half of a byte is exactly 16*q in two's complement), feeds two
// v_mfma_i32_32x32x32_i8 per fragment pair (one group), converts the exact integer result
// (256 * D_g) to fp32 and accumulates sa * sw / 256 * D in fp32.  Both operands use the
// same nibble -> byte -> MFMA-slot order, so each MFMA pairs equal channels.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

constexpr int BM = 128, BN = 128, kThreads = 256;
constexpr int kRowBytes = 48;

struct Smem {
    uint8_t a[2][BM * kRowBytes];
    uint8_t b[2][BN * kRowBytes];
    float sa[2][BM];
    float sw[2][BN];
};

// 8 packed bytes (16 codes) -> one 16-byte int8 MFMA operand holding 16*q per byte.
__device__ __forceinline__ i32x4 expand16(uint32_t p0, uint32_t p1) {
    i32x4 r;
    r[0] = (int)((p0 << 4) & 0xF0F0F0F0u);
    r[1] = (int)(p0 & 0xF0F0F0F0u);
    r[2] = (int)((p1 << 4) & 0xF0F0F0F0u);
    r[3] = (int)(p1 & 0xF0F0F0F0u);
    return r;
}

__global__ __launch_bounds__(kThreads) void gemm_int4_v0_kernel(GemmArgs p) {
    __shared__ Smem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, K = p.K, G = K >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const uint8_t* wcodes = (const uint8_t*)p.wcodes;
    const float* ascales = (const float*)p.ascales;
    const float* wscales = (const float*)p.wscales;

    // global -> LDS assignment: one 16-byte half of one row of A and of W per thread,
    // and one scale (threads 0..127: A rows, 128..255: W rows).
    const int lrow = tid >> 1, lhalf = tid & 1;
    const int64_t am = (m0 + lrow < M) ? m0 + lrow : M - 1;
    const int64_t bn = (n0 + lrow < N) ? n0 + lrow : N - 1;
    const uint8_t* ag = acodes + am * (K / 2) + lhalf * 16;
    const uint8_t* bg = wcodes + bn * (K / 2) + lhalf * 16;
    const float* sg;
    if (tid < BM) {
        int64_t r = (m0 + tid < M) ? m0 + tid : M - 1;
        sg = ascales + r * G;
    } else {
        int64_t r = (n0 + tid - BM < N) ? n0 + tid - BM : N - 1;
        sg = wscales + r * G;
    }
    float* sdst0 = tid < BM ? &sm.sa[0][tid] : &sm.sw[0][tid - BM];
    float* sdst1 = tid < BM ? &sm.sa[1][tid] : &sm.sw[1][tid - BM];

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    uint4 ra = *reinterpret_cast<const uint4*>(ag);
    uint4 rb = *reinterpret_cast<const uint4*>(bg);
    float rs = sg[0];
    *reinterpret_cast<uint4*>(&sm.a[0][lrow * kRowBytes + lhalf * 16]) = ra;
    *reinterpret_cast<uint4*>(&sm.b[0][lrow * kRowBytes + lhalf * 16]) = rb;
    *sdst0 = rs;
    __syncthreads();

    const int fr = lane & 31, fh = lane >> 5;
    for (int g = 0; g < G; ++g) {
        const int cur = g & 1;
        if (g + 1 < G) {
            ra = *reinterpret_cast<const uint4*>(ag + (g + 1) * 32);
            rb = *reinterpret_cast<const uint4*>(bg + (g + 1) * 32);
            rs = sg[g + 1];
        }
        i32x4 opa[2][2], opb[2][2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            uint4 pa = *reinterpret_cast<const uint4*>(
                &sm.a[cur][(wm * 64 + f * 32 + fr) * kRowBytes + fh * 16]);
            opa[f][0] = expand16(pa.x, pa.y);
            opa[f][1] = expand16(pa.z, pa.w);
            uint4 pb = *reinterpret_cast<const uint4*>(
                &sm.b[cur][(wn * 64 + f * 32 + fr) * kRowBytes + fh * 16]);
            opb[f][0] = expand16(pb.x, pb.y);
            opb[f][1] = expand16(pb.z, pb.w);
        }
#pragma unroll
        for (int fa = 0; fa < 2; ++fa) {
            float sav[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float4 v = *reinterpret_cast<const float4*>(
                    &sm.sa[cur][wm * 64 + fa * 32 + 8 * q + 4 * fh]);
                sav[4 * q + 0] = v.x;
                sav[4 * q + 1] = v.y;
                sav[4 * q + 2] = v.z;
                sav[4 * q + 3] = v.w;
            }
#pragma unroll
            for (int fb = 0; fb < 2; ++fb) {
                i32x16 d;
#pragma unroll
                for (int e = 0; e < 16; ++e) d[e] = 0;
                d = __builtin_amdgcn_mfma_i32_32x32x32_i8(opa[fa][0], opb[fb][0], d, 0, 0, 0);
                d = __builtin_amdgcn_mfma_i32_32x32x32_i8(opa[fa][1], opb[fb][1], d, 0, 0, 0);
                const float swv = sm.sw[cur][wn * 64 + fb * 32 + fr] * (1.0f / 256.0f);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[fa][fb][e] += (float)d[e] * (sav[e] * swv);
            }
        }
        if (g + 1 < G) {
            *reinterpret_cast<uint4*>(&sm.a[cur ^ 1][lrow * kRowBytes + lhalf * 16]) = ra;
            *reinterpret_cast<uint4*>(&sm.b[cur ^ 1][lrow * kRowBytes + lhalf * 16]) = rb;
            *(cur ? sdst0 : sdst1) = rs;
        }
        __syncthreads();
    }

    // Epilogue: low-rank up-projection on the MFMA (bf16 x bf16 -> fp32, accumulated
    // straight into the output tile), then bias, GELU, store.
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

void launch_gemm_int4(const GemmArgs& a, hipStream_t st) {
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_int4_v0_kernel, grid, dim3(kThreads), 0, st, a);
}

}  // namespace svdq

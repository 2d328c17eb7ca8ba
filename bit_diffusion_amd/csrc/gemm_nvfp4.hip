// gemm_nvfp4.hip -- NVFP4 variant of the W4A4 GEMM (page "Hugging Face 把 Nunchaku 4-bit
// Diffusion 接到 Diffusers", 技术细节 3: svdq_w4a4 with precision nvfp4), with the same
// low-rank / bias / GELU epilogue as the INT4 kernel.
//
//   y[m,n] = S_a S_w sum_k (e_a[m,k] sb_a[m,k/16]) (e_w[n,k] sb_w[n,k/16]) + lowrank + b
//
// gfx950's scaled MFMA takes power-of-two (E8M0) block scales on 32-element blocks, which
// cannot carry NVFP4's E4M3 scales on 16-element blocks.  Instead each E2M1 value (at
// most 2 significant bits) is multiplied by its E4M3 block scale (at most 4 significant
// bits): the product has at most 6 significant bits and lies in [2^-10, 2688], so it is
// exact in f16 (and in bf16).  The operands are dequantized once per pipeline stage into
// LDS and contracted with the 16-bit MFMA in fp32; S_a * S_w is applied in the epilogue.
//
// Fast kernel (gemm_nvfp4_f16_kernel): 256x192 output tile per 512-thread workgroup, 8
// waves as 4 x 2 of 64x96.  Codes and scale bytes go to LDS by LDS DMA in stages of 256
// channels (128 contiguous bytes of codes per row: whole cache lines), double-buffered,
// one barrier per stage.  Each wave converts the operands of its own MFMA fragments per
// 16-channel k-step: v_cvt_scalef32_pk_f16_fp4 (scale 1) turns a code byte into two exact
// f16 values and v_pk_mul_f16 applies the block scale (exact); v_mfma_f32_32x32x16_f16
// contracts.
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

// ---------------------------------------------------------------- fast kernel
constexpr int kFM = 256, kFN = 192, kFThreads = 512;
constexpr int kFK = 256;                        // channels per pipeline stage
// One stage in LDS: codes of every row (128 bytes: 8 chunks of 16 bytes, chunk c of row r
// stored at position c ^ ((r >> 1) & 7) so that a fragment's 32 rows read one chunk
// conflict-free), then the 16 E4M3 scale bytes of every row.  K is a multiple of 256.
constexpr int kCA = kFM * 128, kCB = kFN * 128;             // 32768, 24576
constexpr int kSA = kFM * 16, kSB = kFN * 16;               // 4096, 3072
constexpr int kFStage = kCA + kCB + kSA + kSB;              // 64512
constexpr int kFSmemBytes = 2 * kFStage;                    // 129024
static_assert(kFSmemBytes <= 160 * 1024, "LDS budget");

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void fbarrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) uint8_t flds_u8;

// Global -> LDS copies (LDS DMA): lane l moves 16 (x4) or 4 (dword) bytes from its own
// global address to LDS byte lds + 16 l (+ 4 l).  The s_nop is the wait state an LDS DMA
// needs after an SALU write of M0.  Completion: s_waitcnt vmcnt(0) before the barrier.
__device__ __forceinline__ void fdma_x4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory");
}
__device__ __forceinline__ void fdma_x1(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds) : "memory");
}

// 8 codes (a dword, code 2i in the low nibble of byte i) times the E4M3 scale sc as an
// exact f16 MFMA operand.
__device__ __forceinline__ f16x8 dequant8(uint32_t w, f16x2 sc) {
    const f16x2 h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sc;
    const f16x2 h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sc;
    const f16x2 h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sc;
    const f16x2 h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sc;
    return f16x8{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

__device__ __forceinline__ f16x2 scale_pair(uint32_t sc, int byte) {
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)(sc >> (8 * byte)), 0);
    return f16x2{v, v};
}

__global__ __launch_bounds__(kFThreads, 1) void gemm_nvfp4_f16_kernel(GemmArgs p) {
    extern __shared__ __align__(16) uint8_t fsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, K = p.K;
    const int S = K / kFK;
    const int64_t num_m = (M + kFM - 1) / kFM;
    const int num_n = (N + kFN - 1) / kFN;
    // tiles in row-major order; the workgroups of one XCD (ids congruent mod 8) take a
    // contiguous range of them when the count allows
    int64_t t = blockIdx.x;
    const int64_t nt = num_m * num_n;
    if ((nt & 7) == 0) t = (t & 7) * (nt >> 3) + (t >> 3);
    const int64_t m0 = (t / num_n) * kFM;
    const int n0 = (int)(t % num_n) * kFN;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(flds_u8*)fsm);

    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const uint8_t* wcodes = (const uint8_t*)p.wcodes;
    const uint8_t* ascales = (const uint8_t*)p.ascales;
    const uint8_t* wscales = (const uint8_t*)p.wscales;

    // ---- copies of stage s: 56 code copies (8 rows x 128 bytes each: 32 for A, 24 for B)
    // and 7 scale copies (16 bytes per row, 64 rows each: 4 for A, 3 for B); wave w issues
    // numbers w, w + 8, ...
    auto issue = [&](int s) {
        const uint32_t base = lds0 + (s & 1) * kFStage;
        const int kc = s * kFK;                       // first channel of the stage
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int d = wave + 8 * q;
            if (d < 56) {
                const bool isa = d < 32;
                const int j = isa ? d : d - 32;
                const int row = 8 * j + (lane >> 3), pos = lane & 7;
                const int c = pos ^ ((row >> 1) & 7);
                const uint8_t* src = isa ? acodes + min(m0 + row, M - 1) * (K / 2)
                                         : wcodes + (int64_t)min(n0 + row, N - 1) * (K / 2);
                fdma_x4(src + kc / 2 + 16 * c, base + (isa ? 0 : kCA) + 1024 * j);
            } else if (d < 63) {
                const int v = d - 56;                 // 0-3 A, 4-6 B
                const bool isa = v < 4;
                const int row = 64 * (isa ? v : v - 4) + lane;
                const uint8_t* src = isa ? ascales + min(m0 + row, M - 1) * (K / 16)
                                         : wscales + (int64_t)min(n0 + row, N - 1) * (K / 16);
                fdma_x4(src + kc / 16, base + kCA + kCB + (isa ? 1024 * v : kSA + 1024 * (v - 4)));
            }
        }
    };

    f32x16 acc[2][3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    // ---- compute one 64-channel sub-stage u of stage buffer b.  The MFMA contracts any
    // consistent permutation of the channels: for k-step kk, lane half h supplies codes
    // 8 (4h + kk) .. + 7 of the sub-stage, i.e. dword kk of its 16-byte chunk 2u + h, in
    // block 2h + kk / 2.
    const int fr = lane & 31, fh = lane >> 5;
    auto compute = [&](int b, int u) {
        const uint8_t* st = fsm + b * kFStage;
        const int su = 4 * u;   // this sub-stage's 4 scale bytes within the row's 16
        uint4 ca[2], cb[3];
        f16x2 sa[2][2], sb[3][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = wm * 64 + 32 * i + fr;
            ca[i] = *reinterpret_cast<const uint4*>(st + row * 128 + 16 * ((2 * u + fh) ^ ((row >> 1) & 7)));
            const uint32_t sc = *reinterpret_cast<const uint32_t*>(st + kCA + kCB + 16 * row + su);
            sa[i][0] = scale_pair(sc, 2 * fh);
            sa[i][1] = scale_pair(sc, 2 * fh + 1);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int row = wn * 96 + 32 * j + fr;
            cb[j] = *reinterpret_cast<const uint4*>(st + kCA + row * 128 + 16 * ((2 * u + fh) ^ ((row >> 1) & 7)));
            const uint32_t sc = *reinterpret_cast<const uint32_t*>(st + kCA + kCB + kSA + 16 * row + su);
            sb[j][0] = scale_pair(sc, 2 * fh);
            sb[j][1] = scale_pair(sc, 2 * fh + 1);
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            f16x8 a[2], bb[3];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint32_t w = kk == 0 ? ca[i].x : kk == 1 ? ca[i].y : kk == 2 ? ca[i].z : ca[i].w;
                a[i] = dequant8(w, sa[i][kk >> 1]);
            }
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint32_t w = kk == 0 ? cb[j].x : kk == 1 ? cb[j].y : kk == 2 ? cb[j].z : cb[j].w;
                bb[j] = dequant8(w, sb[j][kk >> 1]);
            }
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- pipeline: two stage buffers; stage s + 1 is copied while stage s computes
    issue(0);
    for (int s = 0; s < S; ++s) {
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0): this wave's copies of s landed
        fbarrier();                           // every wave's have; buffer (s + 1) & 1 is free
        if (s + 1 < S) issue(s + 1);
#pragma unroll
        for (int u = 0; u < 4; ++u) compute(s & 1, u);
    }

    // ---- epilogue: S_a S_w, low-rank branch, bias, GELU, store
    const float sasw = p.Sa * p.Sw;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] *= sasw;
    const uint16_t* lora = (const uint16_t*)p.lora;
    const uint16_t* l2 = (const uint16_t*)p.l2;
    const int r = p.r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t mrow = min(m0 + wm * 64 + i * 32 + fr, M - 1);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int ncol = min(n0 + wn * 96 + j * 32 + fr, N - 1);
            for (int kk = 0; kk < r; kk += 16) {
                const uint4 va = *reinterpret_cast<const uint4*>(lora + mrow * r + kk + 8 * fh);
                const uint4 vb = *reinterpret_cast<const uint4*>(l2 + (int64_t)ncol * r + kk + 8 * fh);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(vb), acc[i][j], 0, 0, 0);
            }
        }
    }
    const uint16_t* bias = (const uint16_t*)p.bias;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int col = n0 + wn * 96 + j * 32 + fr;
        const bool cok = col < N;
        const float bv = (bias && cok) ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                float v = acc[i][j][e] + bv;
                if (p.act == 1) v = gelu_tanh(v);
                if (cok && row < M) {
                    if (p.out_bf16) ((uint16_t*)p.out)[row * N + col] = (uint16_t)f32_to_bf16(v);
                    else ((float*)p.out)[row * N + col] = v;
                }
            }
    }
}

}  // namespace

bool gemm_nvfp4_init() {
    static int ok = -1;
    if (ok < 0)
        ok = hipFuncSetAttribute((const void*)gemm_nvfp4_f16_kernel,
                                 hipFuncAttributeMaxDynamicSharedMemorySize, kFSmemBytes) == hipSuccess;
    return ok == 1;
}

void launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st) {
    // The fast kernel copies 16-byte pieces of codes and scales: K a multiple of 256 and
    // 16-byte aligned arrays.
    const bool fast = a.K % kFK == 0 && (reinterpret_cast<uintptr_t>(a.acodes) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.wcodes) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.ascales) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.wscales) % 16) == 0;
    const int64_t num_m = (a.M + kFM - 1) / kFM;
    const int num_n = (a.N + kFN - 1) / kFN;
    if (fast && num_m * num_n < ((int64_t)1 << 31) && gemm_nvfp4_init()) {
        hipLaunchKernelGGL(gemm_nvfp4_f16_kernel, dim3((unsigned)(num_m * num_n)), dim3(kFThreads),
                           kFSmemBytes, st, a);
        return;
    }
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_nvfp4_v0_kernel, grid, dim3(kThreads), 0, st, a);
}

}  // namespace svdq

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
// waves as 4 x 2 of 64x96.  Codes and scale bytes of a 64-channel stage are copied to LDS
// by LDS DMA, three stages deep.  Per stage every thread converts one 32-code half row of
// A (and of B for threads < 384): v_cvt_scalef32_pk_f16_fp4 (scale 1) turns a code byte
// into two exact f16 values and v_pk_mul_f16 applies the block scale (exact).  The f16
// rows go to a double-buffered, XOR-swizzled LDS tile and v_mfma_f32_32x32x16_f16
// contracts.  One barrier per stage.
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
constexpr int kFM = 256, kFN = 192, kFK = 64, kFThreads = 512;
// f16 tile of one stage: rows of 64 values (128 bytes), 16-byte chunk c of row r stored at
// chunk position c ^ (r & 7) so that 32 consecutive rows read one chunk conflict-free.
constexpr int kFTile = (kFM + kFN) * 128;                      // 57344 bytes
// raw stage as copied from global memory: codes (row r, 16-byte half h at slot 2r + h), then
// the scale dword of every row
constexpr int kRawA = kFM * 32, kRawB = kFN * 32;               // 8192, 6144
constexpr int kRawSA = kFM * 4, kRawSB = kFN * 4;               // 1024, 768
constexpr int kRaw = kRawA + kRawB + kRawSA + kRawSB;           // 16128
constexpr int kRawStages = 3;
constexpr int kFSmemBytes = 2 * kFTile + kRawStages * kRaw;     // 163072
static_assert(kFSmemBytes <= 160 * 1024, "LDS budget");

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

template <int n>
__device__ __forceinline__ void fwait_vm() {
    static_assert(n >= 0 && n < 16, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0070 | n);   // vmcnt = n, lgkmcnt = 0 (expcnt not waited)
}

__device__ __forceinline__ void fbarrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) uint8_t flds_u8;

// Global -> LDS copies (LDS DMA): lane l moves 16 (x4) or 4 (dword) bytes from its own
// global address to LDS byte lds + 16 l (+ 4 l).  The s_nop is the wait state an LDS DMA
// needs after an SALU write of M0.  Completion is tracked with fwait_vm.
__device__ __forceinline__ void fdma_x4(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds) : "memory");
}
__device__ __forceinline__ void fdma_x1(const void* g, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 :: "v"(g), "s"(lds) : "memory");
}

// 32 codes (16 bytes, code 2i in the low nibble of byte i) times the E4M3 scales sc0 (codes
// 0-15) and sc1 (16-31): 32 exact f16 products, returned as 16 words.
__device__ __forceinline__ void dequant32h(uint4 c, uint32_t sc, uint32_t (&o)[16]) {
    const _Float16 s0 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sc, 0);
    const _Float16 s1 = (_Float16)__builtin_amdgcn_cvt_f32_fp8((int)sc, 1);
    const f16x2 v0 = {s0, s0}, v1 = {s1, s1};
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        f16x2 h;
        switch (i & 3) {
            case 0: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i >> 2], 1.0f, 0); break;
            case 1: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i >> 2], 1.0f, 1); break;
            case 2: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i >> 2], 1.0f, 2); break;
            default: h = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w[i >> 2], 1.0f, 3); break;
        }
        h = h * (i < 8 ? v0 : v1);
        o[i] = __builtin_bit_cast(uint32_t, h);
    }
}

__global__ __launch_bounds__(kFThreads, 1) void gemm_nvfp4_f16_kernel(GemmArgs p) {
    extern __shared__ __align__(16) uint8_t fsm[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, K = p.K, S = K / kFK;
    const int64_t num_m = (M + kFM - 1) / kFM;
    const int num_n = (N + kFN - 1) / kFN;
    // tiles in row-major order, workgroups of one XCD (ids congruent mod 8) on a contiguous
    // range of them when the count allows
    int64_t t = blockIdx.x;
    const int64_t nt = num_m * num_n;
    if ((nt & 7) == 0) t = (t & 7) * (nt >> 3) + (t >> 3);
    const int64_t m0 = (t / num_n) * kFM;
    const int n0 = (int)(t % num_n) * kFN;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(flds_u8*)fsm);
    const uint32_t raw0 = lds0 + 2 * kFTile;

    // ---- copy issue: 21 DMAs per stage, wave w takes numbers w, w + 8, w + 16 (< 21):
    // 0-7 A codes, 8-13 B codes, 14-17 A scales, 18-20 B scales
    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const uint8_t* wcodes = (const uint8_t*)p.wcodes;
    const uint8_t* ascales = (const uint8_t*)p.ascales;
    const uint8_t* wscales = (const uint8_t*)p.wscales;
    auto issue_one = [&](int d, int s, uint32_t raw) {
        if (d < 8) {                      // A codes, slots 64 d + lane
            const int slot = 64 * d + lane, row = slot >> 1;
            const int64_t m = min(m0 + row, M - 1);
            fdma_x4(acodes + m * (K / 2) + s * 32 + 16 * (slot & 1), raw + 1024 * d);
        } else if (d < 14) {              // B codes
            const int slot = 64 * (d - 8) + lane, row = slot >> 1;
            const int n = min(n0 + row, N - 1);
            fdma_x4(wcodes + (int64_t)n * (K / 2) + s * 32 + 16 * (slot & 1), raw + kRawA + 1024 * (d - 8));
        } else if (d < 18) {              // A scales, rows 64 (d - 14) + lane
            const int64_t m = min(m0 + 64 * (d - 14) + lane, M - 1);
            fdma_x1(ascales + m * (K / 16) + s * 4, raw + kRawA + kRawB + 256 * (d - 14));
        } else {                          // B scales
            const int n = min(n0 + 64 * (d - 18) + lane, N - 1);
            fdma_x1(wscales + (int64_t)n * (K / 16) + s * 4, raw + kRawA + kRawB + kRawSA + 256 * (d - 18));
        }
    };
    // DMAs per stage of this wave: 3 for waves 0-4, 2 for waves 5-7
    auto issue = [&](int s) {
        const uint32_t raw = raw0 + (s % kRawStages) * kRaw;
        issue_one(wave, s, raw);
        issue_one(wave + 8, s, raw);
        if (wave + 16 < 21) issue_one(wave + 16, s, raw);
    };

    // ---- conversion: thread t converts half (t & 1) of A row t >> 1 and, for t < 384, of
    // B row t >> 1, from the raw stage to the f16 tile
    const int lr = tid >> 1, lh = tid & 1;
    auto convert_one = [&](const uint8_t* codes, const uint8_t* sc4, uint8_t* row) {
        const uint4 c = *reinterpret_cast<const uint4*>(codes);
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(sc4) >> (16 * lh);
        uint32_t o[16];
        dequant32h(c, sc, o);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<uint4*>(row + 16 * ((4 * lh + q) ^ (lr & 7))) =
                make_uint4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    };
    auto convert = [&](int s, int buf) {
        const uint8_t* raw = fsm + 2 * kFTile + (s % kRawStages) * kRaw;
        uint8_t* tile = fsm + buf * kFTile;
        convert_one(raw + 16 * tid, raw + kRawA + kRawB + 4 * lr, tile + lr * 128);
        if (tid < 2 * kFN)
            convert_one(raw + kRawA + 16 * tid, raw + kRawA + kRawB + kRawSA + 4 * lr, tile + (kFM + lr) * 128);
    };

    f32x16 acc[2][3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int fr = lane & 31, fh = lane >> 5;
    auto compute = [&](int buf) {
        const uint8_t* A = fsm + buf * kFTile + (wm * 64 + fr) * 128;
        const uint8_t* B = fsm + buf * kFTile + (kFM + wn * 96 + fr) * 128;
        const int sw = fr & 7;   // rows of a fragment start at multiples of 8
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int pos = 16 * ((2 * kk + fh) ^ sw);
            f16x8 a[2], b[3];
#pragma unroll
            for (int i = 0; i < 2; ++i) a[i] = *reinterpret_cast<const f16x8*>(A + i * 32 * 128 + pos);
#pragma unroll
            for (int j = 0; j < 3; ++j) b[j] = *reinterpret_cast<const f16x8*>(B + j * 32 * 128 + pos);
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    };

    // ---- pipeline: raw stages s+1, s+2 in flight while stage s computes; per stage one
    // barrier, after which stage s+1 is converted into the other f16 buffer and the copies of
    // stage s+3 go into the raw buffer stage s just released.
    issue(0);
    if (S > 1) issue(1);
    if (S > 2) issue(2);
    fwait_vm<0>();
    fbarrier();
    convert(0, 0);
    for (int s = 0; s < S; ++s) {
        // this wave's copies of stage s + 1 have landed: at most stage s + 2's (2 or 3) remain
        if (s + 2 < S) fwait_vm<2>();
        else fwait_vm<0>();
        fbarrier();   // every wave's have; stage s's f16 tile is complete; raw s is free
        if (s + 3 < S) issue(s + 3);
        if (s + 1 < S) convert(s + 1, (s + 1) & 1);
        compute(s & 1);
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
    // The fast kernel reads 16-byte code pieces and the 4 scale bytes of a row's stage.
    const bool fast = (reinterpret_cast<uintptr_t>(a.acodes) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.wcodes) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.ascales) % 4) == 0 &&
                      (reinterpret_cast<uintptr_t>(a.wscales) % 4) == 0;
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

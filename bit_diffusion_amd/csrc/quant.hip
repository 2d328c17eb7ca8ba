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
// Work mapping: a block of 8 waves owns 16 token rows and walks K in steps of 128 channels
// (two 64-channel groups); wave w takes steps w, w+8, ...  Lane l holds row l % 16 and the
// 32 consecutive channels 32 (l / 16) .. +31 of the step, i.e. one half of one group: the
// lane of one FP6 MFMA fragment, so its 32 codes convert to the fragment's six dwords in a
// single v_cvt_scalef32_2xpk16_fp6_f32.  The group absmax is a max over the lane's 32
// values and its partner lane l ^ 16.  For the low-rank down-projection the same registers
// are the A operands of four v_mfma_f32_16x16x32_bf16 per 16 ranks (the MFMA contracts any
// consistent permutation of the channels; L1 is loaded in the matching order).  The packed
// mode reads L1 prepacked in that lane order (prepack_l1_kernel below), one contiguous 1 KiB
// per operand and wave; the nibble modes read the row-major [r, K] factor, 16 rows a load.
//
// A wave issues the loads of up to kAhead steps at once, in straight-line code, so every
// step waits only for its own data.  smooth_inv goes through a wave-private LDS slice (one
// 128-float slice per step), which needs no barrier.
#include "common.hpp"
#include "launch.hpp"
#include "packed_layout.hpp"
#include "quant_lane.hpp"

// The quantizer is defined as a sequence of individually rounded fp32 operations.
#pragma clang fp contract(off)

namespace svdq {
namespace {

using namespace lane;

constexpr int kRows = 16;
constexpr int kQWaves = 8;
constexpr int kQThreads = kQWaves * 64;
constexpr int kStep = 128;   // channels per wave step

enum Mode { kInt4Nibbles = 0, kInt4Packed = 1, kNvfp4Nibbles = 2 };

// Steps in flight per wave: the register budget (256 VGPRs at 8 waves per block) holds
// three stages up to rank 32 (at rank 32 the third stage's L1 slice is loaded only after
// the first stage is done, into the registers that stage freed) and one beyond; above
// rank 64 the L1 slice is loaded when it is used.
template <int RB>
constexpr int kAhead = RB <= 2 ? 3 : 1;
template <int RB>
constexpr bool kPrefetchL1 = RB <= 4;
template <int RB>
constexpr bool kLateL1 = RB == 2;


template <int RB>
struct Stage {
    uint4 x[4];                                          // 32 bf16: channels 8t .. 8t+7 in x[t]
    uint4 l1[kPrefetchL1<RB> && RB > 0 ? 4 * RB : 1];    // L1 row (16 b + l % 16), same channels
};

// Where the lane's L1 operands live.  Row-major [r, K]: row 16 b + l % 16 (`base` points at
// row l % 16), channels k0 + 8 t.  Prepacked: unit (c, b, t), lane l (`base` points at the
// lane's 16 bytes of unit 0).
template <int MODE>
struct L1Src {
    const uint16_t* base;
    int K;
};

template <int MODE, int RB>
__device__ __forceinline__ uint4 load_l1(const L1Src<MODE>& s, int c, int b, int k0, int t) {
    if constexpr (MODE == kInt4Packed)
        return *reinterpret_cast<const uint4*>(s.base + (((int64_t)c * RB + b) * 4 + t) * 512);
    else
        return *reinterpret_cast<const uint4*>(s.base + (int64_t)b * 16 * s.K + k0 + 8 * t);
}

template <int MODE, int RB>
__device__ __forceinline__ void load_stage_l1(Stage<RB>& st, const L1Src<MODE>& l1s, int c, int k0) {
    if constexpr (kPrefetchL1<RB>)
#pragma unroll
        for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) st.l1[4 * b + t] = load_l1<MODE, RB>(l1s, c, b, k0, t);
}

template <int MODE, int RB>
__device__ __forceinline__ void load_stage(Stage<RB>& st, const uint16_t* xr, const L1Src<MODE>& l1s,
                                           int c, int k0, bool with_l1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) st.x[t] = *reinterpret_cast<const uint4*>(xr + k0 + 8 * t);
    if (with_l1) load_stage_l1<MODE, RB>(st, l1s, c, k0);
}

// x_hat = fp32(x) * smooth_inv for the lane's 32 channels (smooth_inv from the wave's LDS
// slice).
template <int RB>
__device__ __forceinline__ void smooth32(Vals& v, const Stage<RB>& st, const float* si) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float4 s0 = *reinterpret_cast<const float4*>(si + 8 * t);
        const float4 s1 = *reinterpret_cast<const float4*>(si + 8 * t + 4);
        const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        const uint32_t w[4] = {st.x[t].x, st.x[t].y, st.x[t].z, st.x[t].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v.ev[4 * t + i] = __uint_as_float(w[i] << 16) * sv[2 * i];
            v.od[4 * t + i] = __uint_as_float(w[i] & 0xFFFF0000u) * sv[2 * i + 1];
        }
    }
}

template <int RB>
__device__ __forceinline__ void int4_codes32(Vals& v, float s, const Stage<RB>& st,
                                             const float* si) {
    int4_codes32_exact(v, s, [&] { smooth32<RB>(v, st, si); });
}

// Sum the waves' partial low-rank products in a fixed order (wave 0 first) and store bf16
// lora_act: every wave writes its partials, one barrier, then wave w sums its eighth of the
// outputs over the 8 partials.  red holds kQWaves x RB x 256 floats.
template <int RB>
__device__ __forceinline__ void lowrank_finish(f32x4 (&acc)[RB > 0 ? RB : 1], float* red,
                                               int64_t m0, int64_t M, uint16_t* lora) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if constexpr (RB > 0) {
#pragma unroll
        for (int b = 0; b < RB; ++b)
            *reinterpret_cast<f32x4*>(&red[((wave * RB + b) * 64 + lane) * 4]) = acc[b];
        __syncthreads();
        // outputs: RB x 64 lanes x 4 values; this wave takes values e = wave (mod 8)
        constexpr int kOut = RB * 256;
        for (int o = wave * 64 + lane; o < kOut; o += kQWaves * 64) {
            float sum = red[o];
#pragma unroll
            for (int w = 1; w < kQWaves; ++w) sum += red[w * kOut + o];
            const int b = o / 256, l = (o / 4) % 64, i = o % 4;
            const int64_t m = m0 + 4 * (l >> 4) + i;
            if (m < M) lora[m * (RB * 16) + b * 16 + (l & 15)] = (uint16_t)f32_to_bf16(sum);
        }
    }
}

// Quantize and store the lane's 32 channels (half h of group g) of one row.
template <int MODE, int RB>
__device__ __forceinline__ void quantize_half(const Stage<RB>& st, const float* si, int64_t row,
                                              bool row_ok, int g, int h, int G, int K,
                                              const QuantArgs& p) {
    Vals v;
    smooth32<RB>(v, st, si);
    if constexpr (MODE != kNvfp4Nibbles) {
        float a = absmax32(v);
        a = fmaxf(a, __shfl_xor(a, 16, 64));   // the group's other half
        const float s = a / 7.0f;
        int4_codes32<RB>(v, s, st, si);
        if constexpr (MODE == kInt4Nibbles) {
            uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t pair = ((uint32_t)(int)v.ev[i] & 15u) | (((uint32_t)(int)v.od[i] & 15u) << 4);
                d[i >> 2] |= pair << (8 * (i & 3));
            }
            if (row_ok) {
                *reinterpret_cast<uint4*>((uint8_t*)p.codes + row * (K / 2) + g * 32 + h * 16) =
                    make_uint4(d[0], d[1], d[2], d[3]);
                if (h == 0) reinterpret_cast<float*>(p.scales)[row * G + g] = s;
            }
        } else {
            // fields 2i <- channel 2i, 2i+1 <- channel 2i+1; value q / 8 (exact)
            const u32x6 f = cvt_fp6x32(v.ev, v.od, 8.0f);
            const int r32 = (int)(row & 31), L = r32 + 32 * h;
            uint8_t* blk = (uint8_t*)p.codes + packed::act_block(row, g, G);
            *reinterpret_cast<uint4*>(blk + packed::frag_dword(L, 0)) = make_uint4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<uint2*>(blk + packed::frag_dword(L, 4)) = make_uint2(f[4], f[5]);
            if (h == 0) {
                *reinterpret_cast<uint2*>(blk + packed::kFrag + 8 * r32) = packed::act_scale_pair(s);
                if (row_ok && p.scales) reinterpret_cast<float*>(p.scales)[row * G + g] = s;
            }
        }
    } else {
        // NVFP4: the lane's 32 channels are two blocks of 16
        uint32_t d[4], sbs;
        nvfp4_codes32(v, p.S, d, sbs);
        if (row_ok) {
            const int k0 = g * 64 + h * 32;
            uint8_t* sp = (uint8_t*)p.scales + row * (K / 16) + k0 / 16;
            sp[0] = (uint8_t)sbs;
            sp[1] = (uint8_t)(sbs >> 8);
            *reinterpret_cast<uint4*>((uint8_t*)p.codes + row * (K / 2) + k0 / 2) =
                make_uint4(d[0], d[1], d[2], d[3]);
        }
    }
}

template <int RB, int MODE>
__global__ __launch_bounds__(kQThreads) void quant_act_kernel(QuantArgs p) {
    constexpr int NA = kAhead<RB>;
    __shared__ __align__(16) float red[kQWaves * (RB > 0 ? RB : 1) * 256];
    __shared__ __align__(16) float si_lds[kQWaves][NA][kStep];
    const int K = p.K, G = K >> 6;
    const int64_t M = p.M;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t m0 = (int64_t)blockIdx.x * kRows;
    const int rl = lane & 15, q4 = lane >> 4;   // row, quarter of the step
    const int64_t row = m0 + rl;
    const bool row_ok = row < M;
    const uint16_t* xr = (const uint16_t*)p.x + (row_ok ? row : M - 1) * (int64_t)K;
    const L1Src<MODE> l1s{(const uint16_t*)p.l1 + (MODE == kInt4Packed ? 8 * lane : (int64_t)rl * K), K};
    const int nc = (G + 1) >> 1;                                       // steps over K
    const int nsw = nc > wave ? (nc - wave + kQWaves - 1) / kQWaves : 0;  // this wave's steps
    f32x4 acc[RB > 0 ? RB : 1];
#pragma unroll
    for (int b = 0; b < (RB > 0 ? RB : 1); ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int it0 = 0; it0 < nsw; it0 += NA) {
        // loads of up to NA steps, unconditional (clamped) so the waits stay exact
        uint2 siv[NA];
        Stage<RB> st[NA];
#pragma unroll
        for (int s = 0; s < NA; ++s) {
            const int c = wave + kQWaves * min(it0 + s, nsw - 1);
            siv[s] = *reinterpret_cast<const uint2*>(p.smooth_inv + min(c * kStep + 2 * lane, K - 2));
        }
#pragma unroll
        for (int s = 0; s < NA; ++s) {
            const int c = wave + kQWaves * min(it0 + s, nsw - 1);
            load_stage<MODE, RB>(st[s], xr, l1s, c, min(c * kStep + 32 * q4, K - 32),
                                 !(kLateL1<RB> && s == NA - 1));
        }
#pragma unroll
        for (int s = 0; s < NA; ++s) *reinterpret_cast<uint2*>(&si_lds[wave][s][2 * lane]) = siv[s];
#pragma unroll
        for (int s = 0; s < NA; ++s) {
            if (it0 + s < nsw) {
                const int c = wave + kQWaves * (it0 + s);
                const int g = 2 * c + (q4 >> 1), h = q4 & 1;
                const bool g_ok = g < G;   // the last step of an odd group count is half full
                if (!(row_ok && g_ok)) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) st[s].x[t] = make_uint4(0u, 0u, 0u, 0u);
                }
                const float* si = &si_lds[wave][s][32 * q4];
                if (g_ok && (MODE == kInt4Packed || row_ok))
                    quantize_half<MODE, RB>(st[s], si, row, row_ok, g, h, G, K, p);
                if constexpr (RB > 0) {
                    const int k0 = min(c * kStep + 32 * q4, K - 32);
#pragma unroll
                    for (int b = 0; b < RB; ++b)
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            uint4 w;
                            if constexpr (kPrefetchL1<RB>) w = st[s].l1[4 * b + t];
                            else w = load_l1<MODE, RB>(l1s, c, b, k0, t);
                            acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(st[s].x[t]), as_bf16x8(w), acc[b], 0, 0, 0);
                        }
                }
            }
            if (kLateL1<RB> && s == 0) {   // the last stage's L1 slice, into stage 0's registers
                const int c = wave + kQWaves * min(it0 + NA - 1, nsw - 1);
                load_stage_l1<MODE, RB>(st[NA - 1], l1s, c, min(c * kStep + 32 * q4, K - 32));
            }
        }
    }
    lowrank_finish<RB>(acc, red, m0, M, (uint16_t*)p.lora);
}

// Prepacked L1: the low-rank factor [r, K] (bf16) in the lane order of the B operands of
// the packed mode's v_mfma_f32_16x16x32_bf16, so every operand load is one contiguous 1 KiB
// per wave.  Unit (c, b, t) = 128-channel step c, rank block b (ranks 16 b .. 16 b + 15),
// slice t (0..3); lane L of a unit holds the 8 bf16 L1[16 b + L % 16][128 c + 32 (L / 16) +
// 8 t + j], j = 0..7, at byte 16 L.  Units are stored in the order [c][b][t]; channels at or
// beyond K (the second half of the last step when K / 64 is odd) hold zeros.  One thread
// per 16-byte lane of a unit.
__global__ __launch_bounds__(256) void prepack_l1_kernel(int RB, int K, int64_t units,
                                                         const uint16_t* __restrict__ l1,
                                                         uint4* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units) return;
    const int L = (int)(i & 63), t = (int)((i >> 6) & 3);
    const int64_t cb = i >> 8;
    const int b = (int)(cb % RB);
    const int64_t c = cb / RB;
    const int64_t k = c * kStep + 32 * (L >> 4) + 8 * t;
    const int n = 16 * b + (L & 15);
    out[i] = k < K ? *reinterpret_cast<const uint4*>(l1 + (int64_t)n * K + k) : make_uint4(0u, 0u, 0u, 0u);
}

template <int RB, int MODE>
void launch_mode(const QuantArgs& a, int64_t rows, hipStream_t st) {
    hipLaunchKernelGGL((quant_act_kernel<RB, MODE>), dim3((unsigned)((rows + kRows - 1) / kRows)),
                       dim3(kQThreads), 0, st, a);
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

int64_t prepacked_l1_bytes(int r, int K) {
    return (int64_t)((K + kStep - 1) / kStep) * kStep * r * 2;
}

void launch_prepack_l1(int r, int K, const void* l1, void* out, hipStream_t st) {
    const int64_t units = prepacked_l1_bytes(r, K) / 16;
    hipLaunchKernelGGL(prepack_l1_kernel, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, st,
                       r / 16, K, units, (const uint16_t*)l1, (uint4*)out);
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

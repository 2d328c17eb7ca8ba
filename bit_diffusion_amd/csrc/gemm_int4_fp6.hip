// gemm_int4_fp6.hip -- the fast INT4 W4A4 GEMM for gfx950 (prepacked weights).
//
// Same result as svdq_gemm_w4a4 (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
// Diffusers", 技术细节 1 step 4):  y = sum_g sa[m,g] sw[n,g] D_g[m,n] + lora.l2^T + b.
//
// Why FP6.  With 64-channel groups every output needs one fp32 rescale per 64 MACs; on an
// int8 MFMA that is a cvt + mul + fma per output per group, which costs more VALU time than
// the MFMA itself.  Every int4 code q in [-8, 7] is exact in FP6 E2M3 as q/8 (a subnormal,
// sign-magnitude field; |q| = 8 lands on the smallest normal 1.0), the f8f6f4 MFMA runs FP6
// at twice the int8 rate and returns fp32, and v_mfma_scale_f32_32x32x64_f8f6f4 contracts
// exactly one group (K = 64).  So per 32x32 tile and group:
//   R = mfma_fp6(A_g, W_g)                    exact, fp32
//   P = mfma_bf16(sa_hi/lo, sw_hi/lo)         the outer product sa[m] * sw[n] (bf16 hi+lo
//                                             split, relative error ~2^-16)
//   acc = fma(R, P, acc)                      the only VALU work per output and group
//
// Activations arrive as two's-complement nibbles.  Turning a nibble n into the unsigned
// u = n ^ 8 = q + 8 makes its FP6 field simply u zero-extended to 6 bits (u/8 for u < 8 is
// subnormal, u >= 8 is 1.mmm), so the 4 -> 6 bit expansion is shifts and masks (11 VALU ops
// per 16 codes, once per workgroup).  The offset adds 8 * sum_k qw[n,k] per group; its
// contribution -8 sa[m,g] sw[n,g] sum_k qw[n,k] depends on the weights only through
// c[n,g] = -8 sw[n,g] sum_k qw[n,k], which the prepack stores, and is added by one bf16
// MFMA per four groups straight into the accumulator.
//
// Weights are prepacked once (svdq_prepack_weight) into exact signed FP6 fragments in MFMA
// lane order, the bf16 hi/lo scale operands and the correction operands.
//
// Tiling: 256x192 output tile per 512-thread workgroup (8 waves as 4 x 2, each 64x96 =
// 2 x 3 tiles of 32x32), one 64-channel group per pipeline step, operands double-buffered
// in LDS.  Workgroup ids are remapped so the 32 workgroups an XCD runs at once cover a
// compact 4 x 8 block of tiles and share its L2.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

constexpr int BM = 256, BN = 192, kThreads = 512, kStages = 4;
constexpr int kMT = BM / 32;       // A fragments per block
constexpr int kNT = BN / 32;       // W fragments (n-tiles) per block
constexpr int kFragBytes = 1536;   // one 32x64 FP6 fragment: 64 lanes x (16 + 8) bytes
constexpr int kPopBytes = 512;     // 32 columns x 16 bytes: bf16 scale operand (with zeros)
constexpr int kQopBytes = 1024;    // 32 columns x 2 lane halves x 16 bytes
constexpr int kRing = 8;           // scale-operand ring (groups) for the correction MFMA

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Position of the source nibble of dense FP6 field f (0..15) in the 16 codes of two
// dwords (S0 nibbles 0-7, S1 nibbles 8-15): the inverse of spread16().
__device__ __constant__ int8_t kFieldSrc[16] = {0, 1, 3, 4, 6, 7, 9, 10, 12, 13, 15, 8, 2, 11, 5, 14};

// 16 four-bit values (two dwords) -> 16 six-bit fields (three dwords), value zero-extended.
__device__ __forceinline__ void spread16(uint32_t S0, uint32_t S1, uint32_t& T0, uint32_t& T1,
                                         uint32_t& T2) {
    T0 = (S0 & 0x0F00F00Fu) | ((S0 << 2) & 0xC03C03C0u);
    const uint32_t s1s = S1 << 2;
    T1 = (S0 >> 30) | (S1 & 0xF00F00F0u) | (s1s & 0x03C03C00u);
    T2 = (S0 & 0x00F00F00u) | (s1s & 0x3C03C03Cu);
}

// hi = bf16(x), lo = bf16(x - hi); returns hi | lo << 16.
__device__ __forceinline__ uint32_t split_hi_lo(float x) {
    const uint32_t hi = f32_to_bf16(x);
    const uint32_t lo = f32_to_bf16(x - __uint_as_float(hi << 16));
    return hi | (lo << 16);
}

// One group's raw operands, written by global->LDS DMA.
struct Stage {
    uint8_t a_raw[BM * 32];            // packed activation codes, 32 bytes per row
    float sa[BM];                      // activation scales
    uint8_t w_frag[kNT * kFragBytes];  // weight FP6 fragments (prepacked layout)
    uint8_t w_pop[kNT * kPopBytes];    // weight scale operands (prepacked)
};

// One group's activation operands after conversion.
struct Conv {
    uint32_t a_frag[kMT][64][8];       // 6 FP6 dwords per lane (+2 unused)
    uint4 a_pop[BM + 1];               // (d, d, 0, 0), d = sa_hi | sa_lo << 16; last = zeros
};

struct Smem {
    Stage st[kStages];
    Conv cv[2];
    uint32_t a_ring[BM][kRing];        // d per row for the last 8 groups
    uint8_t w_qop[2][kNT * kQopBytes]; // correction operands of the current window
    uint8_t junk[1024];                // target of the padding DMA of waves without qop work
};

// s_waitcnt with vmcnt = n (lgkmcnt = 0): every earlier LDS access of this wave has
// completed and at most n of its vector-memory operations (here: LDS DMA) are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
    __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}

// Workgroup barrier without the memory fence __syncthreads() adds (that fence would wait
// for all in-flight DMA); LDS ordering comes from wait_vm<> before it.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Global -> LDS DMA: each lane moves 16 (dma16) or 4 (dma4) bytes from its own global
// address to lds_wave_base + lane * size.  Issued through asm so that the compiler, which
// cannot tell the DMA targets from the LDS buffers read meanwhile, does not drain every
// DMA in flight before each LDS read; completion is tracked by wait_vm<> instead.  The asm
// writes no VGPR (its result lands in LDS).
typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)p);
}
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(src), "s"(lds_offset(lds_wave_base)) : "memory");
}
__device__ __forceinline__ void dma4(const void* src, void* lds_wave_base) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off"
                 :: "v"(src), "s"(lds_offset(lds_wave_base)) : "memory");
}

__device__ __forceinline__ void tile_coords(int& pid_m, int& pid_n, int num_m, int num_n) {
    const int nt = num_m * num_n;
    int t = blockIdx.x;
    if ((nt & 7) == 0) t = (t & 7) * (nt >> 3) + (t >> 3);   // contiguous tile range per XCD
    const int GM = 4;
    const int group = GM * num_n;
    const int first_m = (t / group) * GM;
    const int gm = min(num_m - first_m, GM);
    const int r = t % group;
    pid_m = first_m + r % gm;
    pid_n = r / gm;
}

__global__ __launch_bounds__(kThreads, 1) void gemm_int4_fp6_kernel(PrepackedGemmArgs p) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, K = p.K, G = K >> 6;
    const int Gp = (G + 3) & ~3;               // groups padded to whole correction windows
    const int NTp = p.ntiles_padded;
    const int num_m = (int)((M + BM - 1) / BM), num_n = (N + BN - 1) / BN;
    int pid_m, pid_n;
    tile_coords(pid_m, pid_n, num_m, num_n);
    const int64_t m0 = (int64_t)pid_m * BM;
    const int n0 = pid_n * BN;
    const int nt0 = pid_n * kNT;               // first n-tile of this block

    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const float* ascales = (const float*)p.ascales;
    const uint8_t* frags = (const uint8_t*)p.prepacked;
    const uint8_t* pops = frags + (int64_t)Gp * NTp * kFragBytes;
    const uint8_t* qops = pops + (int64_t)Gp * NTp * kPopBytes;

    // ---- DMA roles (each wave issues exactly 3 per group, plus 1 at a window start)
    const int64_t a_row = min(m0 + 32 * wave + (lane >> 1), M - 1);
    const uint8_t* a_src = acodes + a_row * (K / 2) + (lane & 1) * 16;
    const int sa_chunk = wave - 4;             // waves 4..7 move 64 scales each
    const int64_t s_row = min(m0 + 64 * (sa_chunk < 0 ? 0 : sa_chunk) + lane, M - 1);
    const float* s_src = ascales + s_row * G;

    auto issue = [&](int h) {
        Stage& S = sm.st[h % kStages];
        const int ha = h < G ? h : G - 1;      // padded groups: any valid address (ignored)
        dma16(a_src + (int64_t)ha * 32, S.a_raw + wave * 1024);
        const uint8_t* wsrc = frags + ((int64_t)h * NTp + nt0) * kFragBytes;
        dma16(wsrc + wave * 1024 + lane * 16, S.w_frag + wave * 1024);
        if (wave == 0) {
            dma16(wsrc + 8 * 1024 + lane * 16, S.w_frag + 8 * 1024);
        } else if (wave < 4) {
            dma16(pops + ((int64_t)h * NTp + nt0) * kPopBytes + (wave - 1) * 1024 + lane * 16,
                  S.w_pop + (wave - 1) * 1024);
        } else {
            dma4(s_src + ha, S.sa + 64 * sa_chunk);
        }
        if ((h & 3) == 0) {
            const uint8_t* qsrc = qops + ((int64_t)(h >> 2) * NTp + nt0) * kQopBytes;
            if (wave < 6) dma16(qsrc + wave * 1024 + lane * 16, sm.w_qop[(h >> 2) & 1] + wave * 1024);
            else dma16(qsrc + lane * 16, sm.junk);
        }
    };

    // ---- activation conversion: raw nibbles -> FP6 fields (u = q + 8), scale operands
    const int crow = tid >> 1, chalf = tid & 1;
    auto convert = [&](int h) {
        const Stage& S = sm.st[h % kStages];
        Conv& C = sm.cv[h & 1];
        uint4 raw = h < G ? *reinterpret_cast<const uint4*>(S.a_raw + crow * 32 + chalf * 16)
                          : make_uint4(0u, 0u, 0u, 0u);
        uint32_t t0, t1, t2, t3, t4, t5;
        spread16(raw.x ^ 0x88888888u, raw.y ^ 0x88888888u, t0, t1, t2);
        spread16(raw.z ^ 0x88888888u, raw.w ^ 0x88888888u, t3, t4, t5);
        uint32_t* dst = C.a_frag[crow >> 5][(crow & 31) + 32 * chalf];
        *reinterpret_cast<uint4*>(dst) = make_uint4(t0, t1, t2, t3);
        *reinterpret_cast<uint2*>(dst + 4) = make_uint2(t4, t5);
        if (tid < BM) {
            const float sav = h < G ? S.sa[tid] : 0.0f;
            const uint32_t d = split_hi_lo(sav);
            C.a_pop[tid] = make_uint4(d, d, 0u, 0u);
            sm.a_ring[tid][h & (kRing - 1)] = d;
        }
    };

    // ---- prologue
    for (int i = tid; i < BM * kRing; i += kThreads) (&sm.a_ring[0][0])[i] = 0u;
    if (tid < 2) sm.cv[tid].a_pop[BM] = make_uint4(0u, 0u, 0u, 0u);
    issue(0);
    if (1 < Gp) issue(1);
    if (2 < Gp) issue(2);
    // wait for groups 0 and 1 (group 2 = 3 DMAs may stay in flight)
    if (2 < Gp) wait_vm<3>(); else wait_vm<0>();
    barrier();
    convert(0);
    barrier();

    f32x16 acc[2][3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int fr = lane & 31, fh = lane >> 5;
    for (int g = 0; g < Gp; ++g) {
        if (g + 3 < Gp) issue(g + 3);
        if (g + 1 < Gp) convert(g + 1);

        const Stage& S = sm.st[g % kStages];
        const Conv& C = sm.cv[g & 1];
        i32x8 aop[2];
        bf16x8 apop[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            aop[i] = *reinterpret_cast<const i32x8*>(C.a_frag[wm * 2 + i][lane]);
            apop[i] = as_bf16x8(C.a_pop[fh ? BM : wm * 64 + i * 32 + fr]);
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int nt = wn * 3 + j;
            const uint8_t* wf = S.w_frag + nt * kFragBytes;
            const uint4 lo = *reinterpret_cast<const uint4*>(wf + lane * 16);
            const uint2 hi = *reinterpret_cast<const uint2*>(wf + 1024 + lane * 8);
            i32x8 wop;
            wop.s0123 = i32x4{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w};
            wop.s45 = (__attribute__((ext_vector_type(2))) int){(int)hi.x, (int)hi.y};
            const uint4 pw = fh ? C.a_pop[BM]
                                : *reinterpret_cast<const uint4*>(S.w_pop + (nt * 32 + fr) * 16);
            const bf16x8 wpop = as_bf16x8(pw);
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const f32x16 r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    aop[i], wop, f32x16{}, 2, 2, 0, 127, 0, 127);
                const f32x16 pp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(apop[i], wpop, f32x16{}, 0, 0, 0);
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = fmaf(r[e], pp[e], acc[i][j][e]);
            }
        }
        if ((g & 3) == 3) {
            // correction for the four groups g-3..g: acc += sum_g sa[m,g] c[n,g]
            const int base = (g - 3) & (kRing - 1);
            const uint8_t* qw = sm.w_qop[(g >> 2) & 1];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const uint4 qa = *reinterpret_cast<const uint4*>(&sm.a_ring[wm * 64 + i * 32 + fr][base]);
#pragma unroll
                for (int j = 0; j < 3; ++j) {
                    const uint4 qb = *reinterpret_cast<const uint4*>(
                        qw + (wn * 3 + j) * kQopBytes + (fr * 2 + fh) * 16);
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), as_bf16x8(qb),
                                                                        acc[i][j], 0, 0, 0);
                }
            }
        }
        // group g+2's DMA must have landed (group g+3's may stay in flight)
        if (g + 3 < Gp) {
            if (((g + 3) & 3) == 0) wait_vm<4>(); else wait_vm<3>();
        } else {
            wait_vm<0>();
        }
        barrier();
    }

    // ---- epilogue: low-rank up-projection on the MFMA, bias, GELU, store
    const uint16_t* lora = (const uint16_t*)p.lora;
    const uint16_t* l2 = (const uint16_t*)p.l2;
    const int r = p.r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t mrow = m0 + wm * 64 + i * 32 + fr;
        if (mrow >= M) mrow = M - 1;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            int ncol = n0 + wn * 96 + j * 32 + fr;
            if (ncol >= N) ncol = N - 1;
            for (int kk = 0; kk < r; kk += 16) {
                const uint4 va = *reinterpret_cast<const uint4*>(lora + mrow * r + kk + 8 * fh);
                const uint4 vb = *reinterpret_cast<const uint4*>(l2 + (int64_t)ncol * r + kk + 8 * fh);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(vb),
                                                                    acc[i][j], 0, 0, 0);
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

// ---------------------------------------------------------------- weight prepack
// One 64-thread block per (group, n-tile); lane l covers column (l % 32) and channel half
// (l / 32) of the group, exactly the B-operand lane of the FP6 MFMA.
__global__ __launch_bounds__(64) void prepack_int4_fp6_kernel(int N, int K, int NTp,
                                                              const uint8_t* __restrict__ wcodes,
                                                              const float* __restrict__ wscales,
                                                              uint8_t* __restrict__ out) {
    const int G = K >> 6, Gp = (G + 3) & ~3;
    const int g = blockIdx.x / NTp, nt = blockIdx.x % NTp;
    const int lane = threadIdx.x, col = lane & 31, half = lane >> 5;
    const int n = nt * 32 + col;
    const bool valid = n < N && g < G;
    uint8_t* frags = out;
    uint8_t* pops = out + (int64_t)Gp * NTp * kFragBytes;
    uint8_t* qops = pops + (int64_t)Gp * NTp * kPopBytes;

    // FP6 fields: field f of this lane holds channel 32*half + 16*(f/16) + src(f % 16),
    // as signed q/8: sign in bit 5, |q| (0..8) in bits 0-4.
    uint32_t w[6] = {0, 0, 0, 0, 0, 0};
    int qsum = 0;
    if (valid) {
        const uint8_t* row = wcodes + (int64_t)n * (K / 2) + g * 32;
        for (int f = 0; f < 32; ++f) {
            const int ch = 32 * half + 16 * (f >> 4) + kFieldSrc[f & 15];
            const uint32_t nib = (row[ch >> 1] >> (4 * (ch & 1))) & 15u;
            const int q = nib >= 8 ? (int)nib - 16 : (int)nib;
            const uint32_t field = (q < 0 ? 32u : 0u) | (uint32_t)(q < 0 ? -q : q);
            const int pos = 6 * f;
            w[pos >> 5] |= field << (pos & 31);
            if ((pos & 31) > 26) w[(pos >> 5) + 1] |= field >> (32 - (pos & 31));
        }
        for (int ch = 0; ch < 64; ++ch) {
            const uint32_t nib = (row[ch >> 1] >> (4 * (ch & 1))) & 15u;
            qsum += nib >= 8 ? (int)nib - 16 : (int)nib;
        }
    }
    uint8_t* fb = frags + ((int64_t)g * NTp + nt) * kFragBytes;
    *reinterpret_cast<uint4*>(fb + lane * 16) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(fb + 1024 + lane * 8) = make_uint2(w[4], w[5]);

    const float sw = valid ? wscales[(int64_t)n * G + g] : 0.0f;
    if (half == 0) {
        const float s64 = sw * 64.0f;   // R = (D + 8 sum qw) / 64
        const uint32_t hi = f32_to_bf16(s64);
        const uint32_t lo = f32_to_bf16(s64 - __uint_as_float(hi << 16));
        *reinterpret_cast<uint4*>(pops + ((int64_t)g * NTp + nt) * kPopBytes + col * 16) =
            make_uint4(hi | (hi << 16), lo, 0u, 0u);
    }
    // correction operand c = -8 sw sum_k qw; half 0 pairs (c_hi, c_hi) with (sa_hi, sa_lo),
    // half 1 pairs (c_lo, 0) with (sa_hi, sa_lo)
    const float c = -8.0f * (float)qsum * sw;
    const uint32_t chi = f32_to_bf16(c);
    const uint32_t clo = f32_to_bf16(c - __uint_as_float(chi << 16));
    const uint32_t word = half == 0 ? (chi | (chi << 16)) : clo;
    uint8_t* qb = qops + ((int64_t)(g >> 2) * NTp + nt) * kQopBytes + (col * 2 + half) * 16 + (g & 3) * 4;
    *reinterpret_cast<uint32_t*>(qb) = word;
}

}  // namespace

int64_t prepacked_int4_bytes(int N, int K) {
    const int64_t G = K / 64, Gp = (G + 3) & ~3LL;
    const int64_t NT = (N + 31) / 32, NTp = (NT + kNT - 1) / kNT * kNT;
    return Gp * NTp * (kFragBytes + kPopBytes) + (Gp / 4) * NTp * kQopBytes;
}

int prepacked_ntiles_padded(int N) {
    const int NT = (N + 31) / 32;
    return (NT + kNT - 1) / kNT * kNT;
}

void launch_prepack_int4(int N, int K, const void* wcodes, const void* wscales, void* out,
                         hipStream_t st) {
    const int G = K / 64, Gp = (G + 3) & ~3;
    const int NTp = prepacked_ntiles_padded(N);
    hipLaunchKernelGGL(prepack_int4_fp6_kernel, dim3(Gp * NTp), dim3(64), 0, st, N, K, NTp,
                       (const uint8_t*)wcodes, (const float*)wscales, (uint8_t*)out);
}

bool gemm_int4_fp6_init() {
    static int ok = -1;
    if (ok < 0)
        ok = hipFuncSetAttribute((const void*)gemm_int4_fp6_kernel,
                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)sizeof(Smem)) == hipSuccess;
    return ok == 1;
}

void launch_gemm_int4_fp6(const PrepackedGemmArgs& a, hipStream_t st) {
    const int num_m = (int)((a.M + BM - 1) / BM), num_n = (a.N + BN - 1) / BN;
    hipLaunchKernelGGL(gemm_int4_fp6_kernel, dim3(num_m * num_n), dim3(kThreads), sizeof(Smem),
                       st, a);
}

}  // namespace svdq

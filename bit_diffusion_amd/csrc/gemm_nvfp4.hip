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
// exact in f16 (and in bf16).  The products are formed in registers right before the
// 16-bit MFMA that contracts them in fp32; S_a * S_w is applied in the epilogue.
//
// Fast kernel (gemm_nvfp4_f16_kernel): 256x192 output tile per 512-thread workgroup, 8
// waves as 4 x 2 of 64x96; one workgroup per CU, each taking every grid-th tile, tiles
// numbered down bands of 4 tile rows.  Codes and scale bytes go to LDS by LDS DMA in stages
// of 256 channels (128 contiguous bytes of codes per row: whole cache lines),
// double-buffered, one barrier per stage.  Each wave converts the operands of its own MFMA
// fragments per 16-channel k-step: v_cvt_scalef32_pk_f16_fp4 (scale 1) turns a code byte
// into two exact f16 values and v_pk_mul_f16 applies the block scale (exact);
// v_mfma_f32_32x32x16_f16 contracts.
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

// Global -> LDS copy (LDS DMA): lane l moves the 16 bytes at base + voff (base wave-uniform,
// in SGPRs; voff the lane's 32-bit byte offset) to LDS byte lds + 16 l, so that a stage's
// advance is one scalar add instead of a 64-bit vector add per copy.  The s_nop is the wait
// state an LDS DMA needs after an SALU write of M0.  Completion: s_waitcnt vmcnt(0) before
// the barrier.
__device__ __forceinline__ void fdma_x4_s(const uint8_t* base, uint32_t voff, uint32_t lds) {
    // readfirstlane returns a signed int: each half goes through uint32_t so that the low
    // half is zero-extended (sign-extended, it would set the high half when bit 31 is set)
    const uint64_t v = (uint64_t)base;
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t b = ((uint64_t)hi << 32) | lo;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"((const uint8_t*)b), "s"(lds) : "memory");
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

// Bytes 2h and 2h + 1 of sc (the two E4M3 block scales lane half h needs in a sub-stage)
// as f16, exact: every E4M3 value is an f16 value, and a scale operand of 1 leaves the
// conversion unscaled.
__device__ __forceinline__ f16x2 scale_pair(uint32_t sc, int h) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sc >> (16 * h), 1.0f, false);
}

// The output tile through LDS: each wave writes its 32 x 96 half-tiles to its own region
// and stores whole 16-byte row segments, non-temporal (the output is written once and read
// by the next layer's kernel).  Row strides keep the two 4-row halves of a 32x32 MFMA
// output on disjoint banks.  A wave's LDS accesses complete in order, so the reads see the
// writes before them and the next half's writes land after them.  N * esz must be a
// multiple of 16 and the output 16-byte aligned.
typedef unsigned nv_u32x4 __attribute__((ext_vector_type(4)));
template <bool kBf16>
__device__ __forceinline__ void store_tile_staged(const f32x16 (&acc)[2][3], uint8_t* smem, const GemmArgs& p,
                                                  int64_t m0, int n0, int wave, int wm, int wn, int lane) {
    constexpr int kEsz = kBf16 ? 2 : 4;
    constexpr int kStride = kBf16 ? 208 : 416;
    constexpr int kSegs = 96 * kEsz / 16;   // 16-byte segments per 96-column row
    static_assert((32 * kSegs) % 64 == 0, "whole segments per lane");
    const int fr = lane & 31, fh = lane >> 5;
    const int64_t M = p.M;
    const int N = p.N;
    uint8_t* stg = smem + wave * (32 * kStride);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                uint8_t* dst = stg + (8 * (e >> 2) + 4 * fh + (e & 3)) * kStride + (j * 32 + fr) * kEsz;
                if constexpr (kBf16) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)f32_to_bf16(acc[i][j][e]);
                else *reinterpret_cast<float*>(dst) = acc[i][j][e];
            }
#pragma unroll
        for (int t = 0; t < 32 * kSegs / 64; ++t) {
            const int c = lane + 64 * t;
            const int lr = c / kSegs, ls = c % kSegs;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + lr * kStride + ls * 16);
            const int64_t row = m0 + wm * 64 + i * 32 + lr;
            const int col = n0 + wn * 96 + ls * (16 / kEsz);
            if (row < M && col < N)
                __builtin_nontemporal_store(nv_u32x4{v.x, v.y, v.z, v.w},
                                            reinterpret_cast<nv_u32x4*>((uint8_t*)p.out + (row * N + col) * kEsz));
        }
    }
}

// Stores per wave of the LDS-staged bf16 epilogue of a whole tile: 2 halves x 6 row segments.
constexpr int kStagedStoresBf16 = 2 * (32 * (96 * 2 / 16) / 64);
static_assert(8 * 32 * 208 <= kFStage, "the bf16 staging area fits in one stage buffer");

// Persistent: workgroup b takes tiles b, b + gridDim.x, ...  With a bf16 output staged
// through LDS, the first stage of the next tile is copied into the free stage buffer while
// the last stage of the current tile computes, and the output goes out through the other
// buffer; the next tile's first wait then lets the epilogue's stores stay in flight (vector
// memory operations complete in issue order, so once at most kStagedStoresBf16 are
// outstanding, the earlier copies have landed).  Other outputs copy the next tile's first
// stage after a barrier, as a new workgroup would.
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
    const int64_t nt = num_m * num_n;
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(flds_u8*)fsm);
    const int esz = p.out_bf16 ? 2 : 4;
    const bool staged = ((int64_t)N * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(p.out) % 16) == 0;
    const bool chain = staged && p.out_bf16;

    const uint8_t* acodes = (const uint8_t*)p.acodes;
    const uint8_t* wcodes = (const uint8_t*)p.wcodes;
    const uint8_t* ascales = (const uint8_t*)p.ascales;
    const uint8_t* wscales = (const uint8_t*)p.wscales;

    // The workgroups of one XCD (ids congruent mod 8) take a contiguous range of tile
    // numbers when the count allows (gridDim.x is a multiple of 8 or nt), and tile numbers
    // run down bands of 4 tile rows, column by column: the 32 tiles an XCD runs at once are
    // then 4 rows x 8 columns, whose operands (1024 A rows, 1536 W rows) its L2 holds
    // once, instead of 1 x 32 (256 A rows, 6144 W rows).
    auto tile_origin = [&](int64_t tile, int64_t& m0, int& n0) {
        int64_t t = tile;
        if ((nt & 7) == 0) t = (t & 7) * (nt >> 3) + (t >> 3);
        constexpr int kBand = 4;
        const int64_t band = t / (kBand * (int64_t)num_n);
        const int64_t first = band * kBand;
        const int64_t rows = min((int64_t)kBand, num_m - first);
        const int64_t in = t - band * kBand * (int64_t)num_n;
        m0 = (first + in % rows) * kFM;
        n0 = (int)(in / rows) * kFN;
    };

    // ---- copies of one stage: 56 code copies (8 rows x 128 bytes each: 32 for A, 24 for
    // B) and 7 scale copies (16 bytes per row, 64 rows each: 4 for A, 3 for B).  Wave w
    // copies code rows 8 j .. 8 j + 7 of A for j = w + 8 q (q < 4) and of B for j = w + 8 q
    // (q < 3), and scale rows 64 w .. of A (w < 4) or 64 (w - 4) .. of B (w = 4..6).  Lane l
    // of a code copy takes row 8 j + l / 8 and stores its chunk c at position l % 8, i.e.
    // chunk c = (l % 8) ^ ((row / 2) % 8), which is the same for every j of the wave.
    const int lrow = lane >> 3;
    const int c16 = 16 * ((lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7));
    // byte offset of each of the wave's copies for a tile (stage 0), from the start of the
    // array it reads (codes of A, codes of W, scales of A for waves 0-3 or of W for 4-6)
    auto tile_off = [&](int64_t m0, int n0, uint32_t (&off)[8]) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
            off[q] = (uint32_t)(min(m0 + 8 * (wave + 8 * q) + lrow, M - 1) * (K / 2) + c16);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            off[4 + q] = (uint32_t)((int64_t)min(n0 + 8 * (wave + 8 * q) + lrow, N - 1) * (K / 2) + c16);
        off[7] = wave < 4 ? (uint32_t)(min(m0 + 64 * wave + lane, M - 1) * (K / 16))
                          : (uint32_t)((int64_t)min(n0 + 64 * (wave - 4) + lane, N - 1) * (K / 16));
    };
    const uint8_t* sbase = wave < 4 ? ascales : wscales;   // this wave's scale copies
    // the copies of the stage starting at channel kc into buffer b
    auto issue = [&](const uint32_t (&off)[8], int kc, int b) {
        const uint32_t base = lds0 + b * kFStage;
        const uint8_t* ab = acodes + kc / 2;
        const uint8_t* wb = wcodes + kc / 2;
#pragma unroll
        for (int q = 0; q < 4; ++q) fdma_x4_s(ab, off[q], base + 1024 * (wave + 8 * q));
#pragma unroll
        for (int q = 0; q < 3; ++q) fdma_x4_s(wb, off[4 + q], base + kCA + 1024 * (wave + 8 * q));
        if (wave < 7) fdma_x4_s(sbase + kc / 16, off[7], base + kCA + kCB + 1024 * wave);
    };

    // ---- compute one 64-channel sub-stage u of stage buffer b.  The MFMA contracts any
    // consistent permutation of the channels: for k-step kk, lane half h supplies codes
    // 8 (4h + kk) .. + 7 of the sub-stage, i.e. dword kk of its 16-byte chunk 2u + h, in
    // block 2h + kk / 2.
    const int fr = lane & 31, fh = lane >> 5;
    f32x16 acc[2][3];
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
            const f16x2 pr = scale_pair(sc, fh);
            sa[i][0] = f16x2{pr[0], pr[0]};
            sa[i][1] = f16x2{pr[1], pr[1]};
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int row = wn * 96 + 32 * j + fr;
            cb[j] = *reinterpret_cast<const uint4*>(st + kCA + row * 128 + 16 * ((2 * u + fh) ^ ((row >> 1) & 7)));
            const uint32_t sc = *reinterpret_cast<const uint32_t*>(st + kCA + kCB + kSA + 16 * row + su);
            const f16x2 pr = scale_pair(sc, fh);
            sb[j][0] = f16x2{pr[0], pr[0]};
            sb[j][1] = f16x2{pr[1], pr[1]};
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

    int gs = 0;                 // stages this workgroup has run (buffer of stage s: (gs + s) & 1)
    bool ahead = false;         // the current tile's first stage is already copied
    bool stores_out = false;    // the previous tile's staged stores may still be in flight
    for (int64_t tile = blockIdx.x; tile < nt; tile += gridDim.x) {
        int64_t m0;
        int n0;
        tile_origin(tile, m0, n0);
        const int64_t next = tile + gridDim.x;
        int64_t nm0 = 0;
        int nn0 = 0;
        if (next < nt) tile_origin(next, nm0, nn0);

#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

        uint32_t src[8];
        tile_off(m0, n0, src);
        if (!ahead) {
            if (tile != blockIdx.x) fbarrier();   // every wave is done with the last epilogue's LDS
            issue(src, 0, gs & 1);
        }
        // ---- pipeline: two stage buffers; stage s + 1 is copied while stage s computes, and
        // when chained the last stage copies the next tile's first
        for (int s = 0; s < S; ++s) {
            if (s == 0 && stores_out)
                __builtin_amdgcn_s_waitcnt(0x0070 | kStagedStoresBf16);   // vmcnt(12), lgkmcnt(0)
            else
                __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0), lgkmcnt(0): this wave's copies of s landed
            fbarrier();                           // every wave's have; buffer (gs + s + 1) & 1 is free
            if (s + 1 < S) {
                issue(src, (s + 1) * kFK, (gs + s + 1) & 1);
            } else if (chain && next < nt) {
                int64_t cm0 = nm0;
                int cn0 = nn0;
                asm volatile("" : "+s"(cm0), "+s"(cn0));   // keeps these addresses out of the loop
                uint32_t nsrc[8];
                tile_off(cm0, cn0, nsrc);
                issue(nsrc, 0, (gs + S) & 1);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) compute((gs + s) & 1, u);
        }
        const int last = (gs + S - 1) & 1;
        ahead = chain && next < nt;
        stores_out = false;
        gs += S;

        // ---- epilogue: S_a S_w, low-rank branch, bias, GELU, store.  Its lane-dependent
        // addresses start from an opaque copy of the lane index, so that they are formed here
        // and not kept in registers through the main loop.
        int el = lane;
        asm volatile("" : "+v"(el));
        const int efr = el & 31, efh = el >> 5;
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
        // the operands of 32 ranks are loaded together, then contracted (per accumulator in
        // rank order), so the loads of a chunk wait for memory once
        const uint16_t* ar[2];
        const uint16_t* br[3];
#pragma unroll
        for (int i = 0; i < 2; ++i) ar[i] = lora + min(m0 + wm * 64 + i * 32 + efr, M - 1) * r + 8 * efh;
#pragma unroll
        for (int j = 0; j < 3; ++j) br[j] = l2 + (int64_t)min(n0 + wn * 96 + j * 32 + efr, N - 1) * r + 8 * efh;
        int kk = 0;
        for (; kk + 32 <= r; kk += 32) {
            uint4 va[2][2], vb[3][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
#pragma unroll
                for (int i = 0; i < 2; ++i) va[i][h] = *reinterpret_cast<const uint4*>(ar[i] + kk + 16 * h);
#pragma unroll
                for (int j = 0; j < 3; ++j) vb[j][h] = *reinterpret_cast<const uint4*>(br[j] + kk + 16 * h);
            }
            __builtin_amdgcn_sched_barrier(0);   // every load issued before the first MFMA
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int j = 0; j < 3; ++j)
#pragma unroll
                    for (int i = 0; i < 2; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[i][h]), as_bf16x8(vb[j][h]),
                                                                          acc[i][j], 0, 0, 0);
        }
        if (kk < r) {   // 16 ranks left
            uint4 va[2], vb[3];
#pragma unroll
            for (int i = 0; i < 2; ++i) va[i] = *reinterpret_cast<const uint4*>(ar[i] + kk);
#pragma unroll
            for (int j = 0; j < 3; ++j) vb[j] = *reinterpret_cast<const uint4*>(br[j] + kk);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int i = 0; i < 2; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va[i]), as_bf16x8(vb[j]), acc[i][j], 0, 0, 0);
        }
        const uint16_t* bias = (const uint16_t*)p.bias;
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int col = n0 + wn * 96 + j * 32 + efr;
            const float bv = (bias && col < N) ? bf16_to_f32(bias[col]) : 0.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    float v = acc[i][j][e] + bv;
                    if (p.act == 1) v = gelu_tanh(v);
                    acc[i][j][e] = v;
                }
        }
        if (staged) {
            fbarrier();   // every wave is done with the last stage's buffer
            if (p.out_bf16) {
                store_tile_staged<true>(acc, fsm + last * kFStage, p, m0, n0, wave, wm, wn, el);
                // a whole tile issues every one of its stores; a partial one may skip some
                stores_out = ahead && m0 + kFM <= M && n0 + kFN <= N;
            } else {
                store_tile_staged<false>(acc, fsm, p, m0, n0, wave, wm, wn, el);
            }
            continue;
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int col = n0 + wn * 96 + j * 32 + efr;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * efh + (e & 3);
                    if (row < M) {
                        if (p.out_bf16) ((uint16_t*)p.out)[row * N + col] = (uint16_t)f32_to_bf16(acc[i][j][e]);
                        else ((float*)p.out)[row * N + col] = acc[i][j][e];
                    }
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
    // the copies address rows by 32-bit byte offsets from the start of each array
    const bool small = a.M * (a.K / 2) < ((int64_t)1 << 31) && (int64_t)a.N * (a.K / 2) < ((int64_t)1 << 31);
    if (fast && small && num_m * num_n < ((int64_t)1 << 31) && gemm_nvfp4_init()) {
        // one workgroup per CU (the LDS of two stage buffers allows no more), each taking
        // every grid-th tile; a multiple of 8 keeps each XCD on its own range of tiles
        const int64_t nt = num_m * num_n;
        const int64_t grid = std::min<int64_t>(nt, std::max(8, cu_count() / 8 * 8));
        hipLaunchKernelGGL(gemm_nvfp4_f16_kernel, dim3((unsigned)grid), dim3(kFThreads), kFSmemBytes, st, a);
        return;
    }
    dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_nvfp4_v0_kernel, grid, dim3(kThreads), 0, st, a);
}

}  // namespace svdq

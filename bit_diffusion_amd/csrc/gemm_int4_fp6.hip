// gemm_int4_fp6.hip -- the fast INT4 W4A4 GEMM for gfx950 on MFMA-ready operands.
//
// Same result as svdq_gemm_w4a4 (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
// Diffusers", 技术细节 1 step 4):  y = sum_g sa[m,g] sw[n,g] D_g[m,n] + lora.l2^T + b,
// D_g the exact integer dot product of group g.
//
// Why FP6.  With 64-channel groups every output needs one fp32 rescale per 64 MACs; on an
// int8 MFMA that is a cvt + mul + fma per output per group, more VALU time than the MFMA.
// Every int4 code is exact in FP6 E2M3 (q / 8), the f8f6f4 MFMA runs FP6 at twice the int8
// rate and returns fp32, and v_mfma_scale_f32_32x32x64_f8f6f4 contracts exactly one group.
// Per 32x32 output tile and group:
//   R = mfma_fp6(A_g, W_g)               = D_g / 64, exact
//   P = mfma_bf16(sa, 64 sw as 3-term bf16 splits) = 64 sa[m] sw[n]  (to a few fp32 ulp)
//   acc = fma(R, P, acc)                 the only VALU work per output and group
// Both operands arrive in the layout of packed_layout.hpp (activations from
// svdq_quantize_act_packed or svdq_pack_act, weights from svdq_prepack_weight), so a
// pipeline stage is a plain copy: 26 KiB per (256x192 tile, group) moved global -> LDS by
// the LDS-DMA path (global_load_lds_dwordx4).  LDS holds a ring of three buffers of two
// groups; while one buffer computes, the next one's copies land and the copies of the one
// after are issued in its first two steps (the barrier that opens a buffer also releases
// the one read before it, which these copies overwrite).
//
// The two groups of a buffer run as one software pipeline of twelve 32x32 sub-tiles: the
// two MFMAs of sub-tile q+1 are issued around the fmas of sub-tile q, across the group
// boundary too, and the second group's operands are read from LDS while the first group's
// last two columns compute.  Copy source addresses are kept in SGPRs.
//
// Tiling: 256x192 output tile per 512-thread workgroup, 8 waves as 4 x 2, each 64x96 =
// 2 x 3 tiles of 32x32 (two waves per SIMD, whose MFMA and VALU work overlap).  Workgroup
// ids are remapped so the workgroups an XCD runs at once cover a compact block of tiles and
// share its L2.  With fp32 output and no activation, a last round of tiles that would fill
// at most a quarter of the GPU is split over K when the caller passes a workspace: each
// split stores its partial tile there and a second kernel adds the splits in a fixed order.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "packed_layout.hpp"
#include "quant_lane.hpp"

namespace svdq {
namespace {

using namespace packed;

constexpr int kThreads = 512, kStages = 6;   // 3 buffers of 2 groups
constexpr int kStageBytes = kAStage + kBStage;   // 26624
constexpr int kAChunks = kAStage / 1024;         // 14
constexpr int kBChunks = kBStage / 1024;         // 12
static_assert(kAStage % 1024 == 0 && kBStage % 1024 == 0, "stages are whole 1 KiB chunks");
static_assert(kAChunks + kBChunks == 26, "chunk assignment below assumes 26 chunks");
constexpr int kSmemBytes = kStages * kStageBytes;

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt with vmcnt = n (lgkmcnt = 0): every earlier LDS access of this wave has
// completed and at most n of its vector-memory operations (here: LDS DMA) are in flight.
template <int n>
__device__ __forceinline__ void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) alone: every earlier LDS access of this wave has completed.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without the memory fence __syncthreads() adds (that fence would wait
// for all in-flight DMA); LDS ordering comes from wait_vm before it.
__device__ __forceinline__ void barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) uint8_t lds_u8;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)p);
}

// Wave-uniform values as SGPR operands of the DMA asm.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const uint8_t*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}
// Global -> LDS DMA of one 1 KiB chunk: lane l moves the 16 bytes at sbase + voff (voff =
// 16 l) to LDS byte address lds + 16 l.  Issued through asm so that the compiler, which
// cannot tell the DMA targets from the LDS buffers read meanwhile, does not drain every
// DMA in flight before each LDS read; completion is tracked by wait_vm instead.  The asm
// writes no VGPR (its result lands in LDS).  An LDS DMA that reads M0 right after an SALU
// write of M0 needs one wait state (the s_nop).
__device__ __forceinline__ void dma_chunk(const uint8_t* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(uniform_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}
// The same with the LDS address given as a wave-uniform base plus a constant, added straight
// into M0 (one SALU instruction instead of an add and a move).
template <uint32_t kOff>
__device__ __forceinline__ void dma_chunk_at(const uint8_t* sbase, uint32_t voff, uint32_t lds_base) {
    asm volatile("s_add_u32 m0, %2, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(uniform_ptr(sbase)), "s"(lds_base), "n"(kOff) : "memory", "scc");
}
// The same under exec & mask (mask 0 or all ones, wave-uniform): with mask 0 no lane
// accesses memory.  Code that waits on these counts them as if they were issued, which is
// exact or one copy too strict either way.
template <uint32_t kOff>
__device__ __forceinline__ void dma_chunk_at_m(const uint8_t* sbase, uint32_t voff, uint32_t lds_base, uint64_t mask) {
    uint64_t saved;
    asm volatile("s_add_u32 m0, %2, %5\n\ts_and_saveexec_b64 %0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %4\n\ts_mov_b64 exec, %0"
                 : "=&s"(saved) : "v"(voff), "s"(lds_base), "s"(uniform_u64(mask)), "s"(uniform_ptr(sbase)), "n"(kOff)
                 : "memory", "scc");
}

// Output tile t (row-major over groups of four tile rows) -> tile coordinates.
__device__ __forceinline__ void tile_of(int t, int& pid_m, int& pid_n, int num_m, int num_n) {
    const int GM = 4;
    const int group = GM * num_n;
    const int first_m = (t / group) * GM;
    const int gm = min(num_m - first_m, GM);
    const int r = t % group;
    pid_m = first_m + r % gm;
    pid_n = r / gm;
}

// Workgroup -> (tile, K split).  Consecutive workgroups go to different XCDs, so block b is
// remapped to give each XCD a contiguous range of tiles.  With a K split (p.nsplit > 1),
// blocks from p.nfull on take the remaining tiles t >= p.nfull in p.nsplit parts of
// p.gsplit groups each.
__device__ __forceinline__ void work_of(const PackedGemmArgs& p, int num_m, int num_n, int& pid_m,
                                        int& pid_n, int& split) {
    const int nt = num_m * num_n;
    int b = blockIdx.x, t;
    split = -1;
    if (p.nsplit > 1 && b >= p.nfull) {
        t = p.nfull + (b - p.nfull) / p.nsplit;
        split = (b - p.nfull) % p.nsplit;
    } else {
        const int n = p.nsplit > 1 ? p.nfull : nt;
        t = (n & 7) == 0 ? (b & 7) * (n >> 3) + (b >> 3) : b;
    }
    tile_of(t, pid_m, pid_n, num_m, num_n);
}

// What the bias loads read when there is no bias.
__device__ const uint16_t kZeroBf16[1] = {0};

// Epilogue staging: each wave writes its 32 x 96 half-tiles to LDS and stores whole
// 16-byte row segments.  Row strides are chosen so that the two 4-row halves of a
// 32x32 MFMA output write disjoint LDS banks.
template <bool kBf16>
constexpr int kStgStride = kBf16 ? 208 : 416;

// The tile as bf16 in LDS for the next layer's quantization: [256 rows][192 columns], row
// stride 400 bytes.
constexpr int kTileStride = 2 * kBN + 16;
// the next layer's operands beside the bf16 tile: l1 (up to rank 128) and smoothing slices
constexpr int kMaxNextRank = 128;
constexpr int kMaxL1Pieces = kMaxNextRank * 24 / kThreads;   // 16-byte pieces per thread
constexpr int kL1SliceOff = kBM * kTileStride;
constexpr int kSiSliceOff = kL1SliceOff + kMaxNextRank * kTileStride;
static_assert(kMaxNextRank * 24 % kThreads == 0, "whole pieces per thread");
static_assert(kSiSliceOff + 4 * kBN <= kSmemBytes, "the slices fit beside the tile");
static_assert(kBM * kTileStride <= kSmemBytes, "the bf16 tile fits in the pipeline buffers");

template <bool kBf16, bool kGelu, bool kNext = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4a4_fp6_kernel(PackedGemmArgs p) {
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t M = p.M;
    const int N = p.N, Gall = p.K >> 6;
    const int num_m = (int)((M + kBM - 1) / kBM), num_n = (N + kBN - 1) / kBN;
    int pid_m, pid_n, split;
    work_of(p, num_m, num_n, pid_m, pid_n, split);
    const int64_t m0 = (int64_t)pid_m * kBM;
    const int n0 = pid_n * kBN;
    // this workgroup's groups: all, or split `split` of a K-split tile
    const int g_begin = split < 0 ? 0 : split * p.gsplit;
    const int G = split < 0 ? Gall : min(Gall - g_begin, p.gsplit);

    const uint8_t* a_base = (const uint8_t*)p.act + ((int64_t)pid_m * Gall + g_begin) * kAStage;
    const uint8_t* b_base = (const uint8_t*)p.wgt + ((int64_t)pid_n * Gall + g_begin) * kBStage;
    const uint32_t lds0 = lds_offset(smem);
    const uint32_t voff = lane * 16;

    // One group's stage (start and tail of the pipeline): chunks 0-13 activations, 14-25
    // weights.  Wave w copies chunks w, w + 8 and w + 16; waves 0 and 1 also 24 and 25.
    auto issue = [&](int h, int slot) {
        const uint8_t* ag = a_base + (int64_t)h * kAStage;
        const uint8_t* bg = b_base + (int64_t)h * kBStage;
        const uint32_t dst = lds0 + slot * kStageBytes;
        dma_chunk(ag + wave * 1024, voff, dst + wave * 1024);
        if (wave + 8 < kAChunks) dma_chunk(ag + (wave + 8) * 1024, voff, dst + (wave + 8) * 1024);
        else dma_chunk(bg + (wave + 8 - kAChunks) * 1024, voff, dst + (wave + 8) * 1024);
        dma_chunk(bg + (wave + 16 - kAChunks) * 1024, voff, dst + (wave + 16) * 1024);
        if (wave < 2) dma_chunk(bg + (wave + 24 - kAChunks) * 1024, voff, dst + (wave + 24) * 1024);
    };

    const int fr = lane & 31, fh = lane >> 5;

    // The low-rank up-projection goes first: acc = lora_act . l2^T.  Its operand loads
    // (and the bias) are issued ahead of the first copies, so their latency hides behind
    // the wait for the first buffers instead of standing in the epilogue.
    const uint16_t* lora = (const uint16_t*)p.lora;
    const uint16_t* l2 = (const uint16_t*)p.l2;
    const int r = split > 0 ? 0 : p.r;   // the low-rank term and the bias go in once per tile
    int64_t mrow[2];
    int ncol[3];
#pragma unroll
    for (int i = 0; i < 2; ++i) mrow[i] = min(m0 + wm * 64 + i * 32 + fr, M - 1);
#pragma unroll
    for (int j = 0; j < 3; ++j) ncol[j] = min(n0 + wn * 96 + j * 32 + fr, N - 1);
    uint4 la[2][2], lb[3][2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
        if (16 * c < r) {
#pragma unroll
            for (int i = 0; i < 2; ++i) la[i][c] = *reinterpret_cast<const uint4*>(lora + mrow[i] * r + 16 * c + 8 * fh);
#pragma unroll
            for (int j = 0; j < 3; ++j) lb[j][c] = *reinterpret_cast<const uint4*>(l2 + (int64_t)ncol[j] * r + 16 * c + 8 * fh);
        }
    // The bias as raw bf16, loaded without a branch (a load under a divergent branch gets
    // a wait for every load in flight right after it); with no bias, or in a K split other
    // than the first, the loads read a zero instead.  Converted in the epilogue.
    const bool has_bias = p.bias != nullptr && split <= 0;
    const uint16_t* bsrc = has_bias ? (const uint16_t*)p.bias : kZeroBf16;
    uint32_t braw[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) braw[j] = bsrc[has_bias ? ncol[j] : 0];

    // Buffer (third) t holds groups 2t and 2t + 1, 52 chunks: chunk c is chunk c % 26 of
    // group 2t + c / 26.  Wave w copies chunks w + 8 j, j = 0..6 (j = 6 exists for w < 4
    // only and is issued under an exec mask, so the loop below has no branches: branches
    // there made the register allocator spill).
    auto chunk_src = [&](int h0, int c) -> const uint8_t* {
        const int k = c >= 26 ? 1 : 0;
        const int cg = c - 26 * k;
        const int h = h0 + k;
        return cg < kAChunks ? a_base + (int64_t)h * kAStage + cg * 1024
                             : b_base + (int64_t)h * kBStage + (cg - kAChunks) * 1024;
    };
    const uint64_t mask_lo4 = uniform_u64((wave < 4) ? ~0ull : 0ull);
    // Source of copy j for third 0 and its advance per third, both wave-uniform (SGPRs):
    // chunk c = wave + 8 j is an activation or a weight chunk depending on the wave only
    // (c is clamped for the masked seventh copy of waves 4-7, which reads nothing).
    uint64_t src0[7];
    uint32_t step[7];
#pragma unroll
    for (int j = 0; j < 7; ++j) {
        const int c = min(wave + 8 * j, 51);
        const int cg = c >= 26 ? c - 26 : c;
        src0[j] = uniform_u64((uint64_t)chunk_src(0, c));
        step[j] = __builtin_amdgcn_readfirstlane(cg < kAChunks ? 2 * kAStage : 2 * kBStage);
    }
    // Copy j of third t: chunk wave + 8 j, at LDS offset base_t + 8 KiB j, base_t the third's
    // buffer plus this wave's first chunk (computed once per third, in an SGPR).
    auto issue_j = [&](int t, auto jc, uint32_t base_t) {   // groups 2t and 2t + 1 both exist
        constexpr int j = decltype(jc)::value;
        const uint8_t* src = (const uint8_t*)(src0[j] + (uint64_t)((uint32_t)t * step[j]));
        if constexpr (j < 6) dma_chunk_at<8192u * j>(src, voff, base_t);
        else dma_chunk_at_m<8192u * j>(src, voff, base_t, mask_lo4);
    };
    for (int h = 0; h < min(G, 4); ++h) issue(h, h);

    f32x16 acc[2][3];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    // the operands above and the first two groups have landed (with four groups issued,
    // at most the 6 or 8 copies of groups 2 and 3 are in flight)
    if (G >= 4) wait_vm<6>();
    else wait_vm<0>();
#pragma unroll
    for (int c = 0; c < 2; ++c)
        if (16 * c < r) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(la[i][c]), as_bf16x8(lb[j][c]),
                                                                        acc[i][j], 0, 0, 0);
        }
    for (int kk = 32; kk < r; kk += 16) {   // ranks beyond 32
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint4 va = *reinterpret_cast<const uint4*>(lora + mrow[i] * r + kk + 8 * fh);
#pragma unroll
            for (int j = 0; j < 3; ++j) {
                const uint4 vb = *reinterpret_cast<const uint4*>(l2 + (int64_t)ncol[j] * r + kk + 8 * fh);
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(va), as_bf16x8(vb), acc[i][j], 0, 0, 0);
            }
        }
    }

    // The operands of this wave for one group: two activation fragments and their scale
    // operands, three weight fragments and theirs.
    struct Frags {
        i32x8 a[2];
        uint2 ax[2];   // the activation scale words: the scale MFMA's A operand as stored
        i32x8 w[3];
        bf16x4 wp[3];
    };
    auto load_frags = [&](const uint8_t* S, Frags& f) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint8_t* Ab = S + (2 * wm + i) * kABlock;
            const uint4 v0 = *reinterpret_cast<const uint4*>(Ab + lane * 16);
            // volatile: a load of its own, straight into the operand's registers (merged
            // with its neighbour it would need two moves)
            const uint64_t v1q = *(const volatile __attribute__((address_space(3))) uint64_t*)(Ab + 1024 + lane * 8);
            const uint2 v1 = make_uint2((uint32_t)v1q, (uint32_t)(v1q >> 32));
            f.ax[i] = *reinterpret_cast<const uint2*>(Ab + kFrag + fr * 8);
            f.a[i].s0123 = i32x4{(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w};
            f.a[i].s45 = (__attribute__((ext_vector_type(2))) int){(int)v1.x, (int)v1.y};
        }
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const uint8_t* Bb = S + kAStage + (3 * wn + j) * kBBlock;
            const uint4 w0v = *reinterpret_cast<const uint4*>(Bb + lane * 16);
            const uint64_t w1q = *(const volatile __attribute__((address_space(3))) uint64_t*)(Bb + 1024 + lane * 8);
            const uint2 w1v = make_uint2((uint32_t)w1q, (uint32_t)(w1q >> 32));
            f.w[j].s0123 = i32x4{(int)w0v.x, (int)w0v.y, (int)w0v.z, (int)w0v.w};
            f.w[j].s45 = (__attribute__((ext_vector_type(2))) int){(int)w1v.x, (int)w1v.y};
            f.wp[j] = __builtin_bit_cast(bf16x4, *reinterpret_cast<const uint2*>(Bb + kFrag + lane * 8));
        }
    };
    // The activation scale operand of the scale-product MFMA: the row's two words (h, h, m, l)
    // serve both halves of the lanes as they are (packed_layout.hpp).
    auto ap_of = [](uint2 x) { return __builtin_bit_cast(bf16x4, x); };
    // Software-pipelined: the two MFMAs of pair q+1 are issued around the fmas of pair q,
    // so the MFMA pipe and the VALU work at the same time within one wave.
    auto compute = [&](const Frags& f) {
        f32x16 r0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[0], f.w[0], f32x16{}, 2, 2, 0, 127, 0, 127);
        f32x16 p0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ap_of(f.ax[0]), f.wp[0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 6; ++q) {
            const int i = q & 1, j = q >> 1;
            f32x16 r1, p1;
            if (q < 5) {
                const int i1 = (q + 1) & 1, j1 = (q + 1) >> 1;
                r1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i1], f.w[j1], f32x16{}, 2, 2, 0, 127, 0, 127);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][j][e] = fmaf(r0[e], p0[e], acc[i][j][e]);
            __builtin_amdgcn_sched_barrier(0);
            if (q < 5) {
                const int i1 = (q + 1) & 1, j1 = (q + 1) >> 1;
                p1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ap_of(f.ax[i1]), f.wp[j1], f32x16{}, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 8; e < 16; ++e) acc[i][j][e] = fmaf(r0[e], p0[e], acc[i][j][e]);
            __builtin_amdgcn_sched_barrier(0);
            r0 = r1;
            p0 = p1;
        }
    };

    // Both groups of a third in one software pipeline of twelve 32x32 sub-tiles (no drain
    // and refill between the groups): the second group's operands are read once the first
    // group is done with its weight columns 0 and 1; `between(q)` runs after steps 0 and 1.
    auto compute2 = [&](const Frags& fa, Frags& fb, const uint8_t* Sb, auto&& between) {
        f32x16 r0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fa.a[0], fa.w[0], f32x16{}, 2, 2, 0, 127, 0, 127);
        f32x16 p0 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ap_of(fa.ax[0]), fa.wp[0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < 12; ++q) {
            const int i = q & 1, j = (q >> 1) % 3;
            const int q1 = q + 1, i1 = q1 & 1, j1 = (q1 >> 1) % 3;
            const Frags& fn = q1 < 6 ? fa : fb;
            f32x16 r1, p1;
            if (q < 11)
                r1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fn.a[i1], fn.w[j1], f32x16{}, 2, 2, 0, 127, 0, 127);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][j][e] = fmaf(r0[e], p0[e], acc[i][j][e]);
            __builtin_amdgcn_sched_barrier(0);
            if (q < 11) p1 = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ap_of(fn.ax[i1]), fn.wp[j1], f32x16{}, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 8; e < 16; ++e) acc[i][j][e] = fmaf(r0[e], p0[e], acc[i][j][e]);
            __builtin_amdgcn_sched_barrier(0);
            if (q == 2) {   // sub-tile 3's MFMAs are issued: the first group's weight
                            // columns 0 and 1 are no longer read
                // The first group's reads have landed by now; waiting for them here keeps
                // the LDS counter (at most 15 in flight) from forcing a wait on the oldest
                // of the 15 reads below instead.
                wait_lgkm0();
                load_frags(Sb, fb);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (q <= 1) {
                between(q);
                __builtin_amdgcn_sched_barrier(0);
            }
            r0 = r1;
            p0 = p1;
        }
    };

    // byte offsets of the buffers of thirds t and t + 2, rotated over the three buffers
    constexpr uint32_t kBuf = 2 * kStageBytes;
    uint32_t off_t = 0, off_t2 = 2 * kBuf;
    const uint32_t lds_w = __builtin_amdgcn_readfirstlane(lds0 + wave * 1024);
    int t = 0;
    for (; 2 * t + 5 < G; ++t) {   // the third two ahead (groups 2t+4, 2t+5) exists
        wait_vm<6>();   // this wave's copies of third t have landed (third t+1's may not)
        barrier();      // every wave's have; third t-1's buffer is no longer read
        const uint8_t* S = smem + off_t;
        {
            Frags f, f1;
            load_frags(S, f);
            // third t+2's copies go into third t-1's buffer, which the barrier above
            // released, early in the third so they have two thirds to land
            const uint32_t base_t = lds_w + off_t2;
            compute2(f, f1, S + kStageBytes, [&](int q) {
                using std::integral_constant;
                if (q == 0) {
                    issue_j(t + 2, integral_constant<int, 0>{}, base_t);
                    issue_j(t + 2, integral_constant<int, 1>{}, base_t);
                    issue_j(t + 2, integral_constant<int, 2>{}, base_t);
                } else {
                    issue_j(t + 2, integral_constant<int, 3>{}, base_t);
                    issue_j(t + 2, integral_constant<int, 4>{}, base_t);
                    issue_j(t + 2, integral_constant<int, 5>{}, base_t);
                    issue_j(t + 2, integral_constant<int, 6>{}, base_t);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        }
        off_t = off_t == 2 * kBuf ? 0u : off_t + kBuf;
        off_t2 = off_t2 == 2 * kBuf ? 0u : off_t2 + kBuf;
    }
    // tail: thirds t and t+1 are issued; at most one group (2t+4 = G-1) is not
    wait_vm<0>();
    barrier();
    for (int h = 2 * t + 4; h < G; ++h) issue(h, h % kStages);
    for (int g = 2 * t; g < min(G, 2 * t + 2); ++g) {
        Frags f;
        load_frags(smem + (g % kStages) * kStageBytes, f);
        compute(f);
    }
    if (2 * t + 2 < G) {
        wait_vm<0>();
        barrier();
        for (int g = 2 * t + 2; g < G; ++g) {
            Frags f;
            load_frags(smem + (g % kStages) * kStageBytes, f);
            compute(f);
        }
    }

    // ---- epilogue: bias, GELU, store
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 3; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                float v = acc[i][j][e] + __uint_as_float(braw[j] << 16);
                if constexpr (kGelu) v = gelu_tanh(v);
                acc[i][j][e] = v;
            }

    if constexpr (kNext) {
        // The next layer's activation kernel on this tile, from the bf16 values this layer
        // would store (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers",
        // 技术细节 1 steps 1, 3, 4 applied to this output): smoothing, 64-channel groups
        // (the tile's 192 columns are three whole groups), codes and scales in the packed
        // layout, and this tile's share of the next low-rank down-projection.
        static_assert(kBf16, "the next layer reads bf16");
        const int G2 = N >> 6;                    // the next layer's groups
        const int ngr = min(3, (N - n0) >> 6);    // whole groups in this tile
        const int R2 = p.next_r;
        const int tid = threadIdx.x;
        // the tile's slices of the next layer's smoothing factors and l1 (rows of R2, this
        // tile's channels), loaded into registers now so their latency overlaps the tile's
        // store to LDS, and stored next to it after the barrier
        const uint16_t* l1n = (const uint16_t*)p.next_l1;
        const int nl1 = R2 * 24;                  // 16-byte pieces of the l1 slice
        uint4 l1v[kMaxL1Pieces];
#pragma unroll
        for (int k = 0; k < kMaxL1Pieces; ++k) {
            const int idx = tid + kThreads * k, jr = idx / 24, c8 = idx - 24 * jr;
            l1v[k] = idx < nl1 && c8 < 8 * ngr
                         ? *reinterpret_cast<const uint4*>(l1n + (int64_t)jr * N + n0 + 8 * c8)
                         : make_uint4(0u, 0u, 0u, 0u);
        }
        const float4 siv = tid < 16 * ngr ? *reinterpret_cast<const float4*>(p.next_si + n0 + 4 * tid)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
        barrier();   // every wave is done with the pipeline buffers
        uint8_t* tl = smem;
        uint8_t* l1t = smem + kL1SliceOff;
        float* sil = reinterpret_cast<float*>(smem + kSiSliceOff);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 3; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int rr = wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                    const int cc = wn * 96 + j * 32 + fr;
                    *reinterpret_cast<uint16_t*>(tl + rr * kTileStride + 2 * cc) =
                        (uint16_t)f32_to_bf16(acc[i][j][e]);
                }
#pragma unroll
        for (int k = 0; k < kMaxL1Pieces; ++k) {
            const int idx = tid + kThreads * k, jr = idx / 24, c8 = idx - 24 * jr;
            if (idx < nl1) *reinterpret_cast<uint4*>(l1t + jr * kTileStride + 16 * c8) = l1v[k];
        }
        if (tid < 48) *reinterpret_cast<float4*>(sil + 4 * tid) = siv;
        barrier();
        // 24 fragments (8 blocks of 32 rows x 3 groups); wave w quantizes rows 32 w .. + 31
        // of each group.  Lane L: row L % 32 of the block, channels 32 (L / 32) .. + 31.
        const int h = lane >> 5, r32 = lane & 31;
        const int rr = wave * 32 + r32;
        const int64_t row = m0 + rr;
#pragma unroll 1
        for (int gi = 0; gi < ngr; ++gi) {
            const int c0 = gi * 64 + 32 * h;
            uint4 xw[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                xw[t] = row < M ? *reinterpret_cast<const uint4*>(tl + rr * kTileStride + 2 * (c0 + 8 * t))
                                : make_uint4(0u, 0u, 0u, 0u);   // padding rows quantize to zero
            lane::Vals v;
            const float* si = sil + c0;
            auto smooth = [&] {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float4 s0 = *reinterpret_cast<const float4*>(si + 8 * t);
                    const float4 s1 = *reinterpret_cast<const float4*>(si + 8 * t + 4);
                    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
                    const uint32_t w[4] = {xw[t].x, xw[t].y, xw[t].z, xw[t].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v.ev[4 * t + i] = __uint_as_float(w[i] << 16) * sv[2 * i];
                        v.od[4 * t + i] = __uint_as_float(w[i] & 0xFFFF0000u) * sv[2 * i + 1];
                    }
                }
            };
            smooth();
            float a = lane::absmax32(v);
            a = fmaxf(a, __shfl_xor(a, 32, 64));   // the group's other half
            const float s = a / 7.0f;
            lane::int4_codes32_exact(v, s, smooth);
            const lane::u32x6 f = lane::cvt_fp6x32(v.ev, v.od, 8.0f);
            const int g2 = (n0 >> 6) + gi;
            uint8_t* blk = (uint8_t*)p.next_packed + act_block(row, g2, G2);
            *reinterpret_cast<uint4*>(blk + frag_dword(lane, 0)) = make_uint4(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<uint2*>(blk + frag_dword(lane, 4)) = make_uint2(f[4], f[5]);
            if (h == 0) {
                *reinterpret_cast<uint2*>(blk + kFrag + 8 * r32) = act_scale_pair(s);
                if (row < M && p.next_scales) p.next_scales[row * G2 + g2] = s;
            }
        }
        // this tile's channels' share of the next layer's lora_act = x . l1^T for rows
        // 32 w .. + 31 (two 16-row MFMA blocks), stored as this tile's fp32 partial sums
        // (slot pid_n of the workspace); a second kernel adds the slots in a fixed order
        if (R2 > 0) {
            const int nks = 2 * ngr;   // 32-channel steps
            const int64_t Mpad = (int64_t)num_m * kBM;
            float* part = p.lora_work + ((int64_t)pid_n * Mpad + m0) * R2;
            uint4 av[2][6];
#pragma unroll
            for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
                for (int ks = 0; ks < 6; ++ks)
                    if (ks < nks)
                        av[rb2][ks] = *reinterpret_cast<const uint4*>(
                            tl + (wave * 32 + rb2 * 16 + (lane & 15)) * kTileStride + 2 * (32 * ks + 8 * (lane >> 4)));
#pragma unroll 1
            for (int jb = 0; jb < R2 / 16; ++jb) {
                f32x4 c[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
                const uint8_t* bl = l1t + (16 * jb + (lane & 15)) * kTileStride + 16 * (lane >> 4);
#pragma unroll
                for (int ks = 0; ks < 6; ++ks)
                    if (ks < nks) {
                        const uint4 bv4 = *reinterpret_cast<const uint4*>(bl + 64 * ks);
#pragma unroll
                        for (int rb2 = 0; rb2 < 2; ++rb2)
                            c[rb2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[rb2][ks]), as_bf16x8(bv4), c[rb2], 0, 0, 0);
                    }
#pragma unroll
                for (int rb2 = 0; rb2 < 2; ++rb2)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rw = wave * 32 + rb2 * 16 + 4 * (lane >> 4) + i;   // tile row (padding rows too)
                        part[(int64_t)rw * R2 + 16 * jb + (lane & 15)] = c[rb2][i];
                    }
            }
        }
        return;
    }
    if constexpr (!kBf16 && !kGelu) {
        if (split >= 0) {
            // A K split: this split's fp32 partial tile goes to its workspace slot in the
            // accumulators' own order (lane-contiguous 16-byte pieces); sum_splits_kernel
            // adds the splits in order 0, 1, ... and stores the tile.
            float* part = p.split_ws + ((int64_t)(blockIdx.x - p.nfull)) * (kBM * kBN);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 3; ++j)
#pragma unroll
                    for (int e4 = 0; e4 < 4; ++e4)
                        *reinterpret_cast<f32x4*>(part + ((((wave * 2 + i) * 3 + j) * 4 + e4) * 64 + lane) * 4) =
                            f32x4{acc[i][j][4 * e4], acc[i][j][4 * e4 + 1], acc[i][j][4 * e4 + 2], acc[i][j][4 * e4 + 3]};
            return;
        }
    }
    constexpr int kEsz = kBf16 ? 2 : 4;
    if (p.vec_store) {
        // rows of 16-byte segments through LDS; N * kEsz is a multiple of 16 here
        constexpr int kStride = kStgStride<kBf16>;
        constexpr int kSegs = 96 * kEsz / 16;   // segments per 96-column row
        barrier();                               // all waves are done with the pipeline stages
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
            // a wave's LDS accesses complete in order: the reads see the writes above, and
            // the next half's writes land after these reads
            static_assert((32 * kSegs) % 64 == 0, "whole segments per lane");
#pragma unroll
            for (int t = 0; t < 32 * kSegs / 64; ++t) {
                const int c = lane + 64 * t;
                const int lr = c / kSegs, ls = c % kSegs;
                const uint4 v = *reinterpret_cast<const uint4*>(stg + lr * kStride + ls * 16);
                const int64_t row = m0 + wm * 64 + i * 32 + lr;
                const int col = n0 + wn * 96 + ls * (16 / kEsz);
                // streaming stores: the output is written once and read by the next
                // layer's kernel, so it need not allocate in the L2 on its way out
                if (row < M && col < N)
                    __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                                reinterpret_cast<u32x4*>((uint8_t*)p.out + (row * N + col) * kEsz));
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < 3; ++j) {
            const int col = n0 + wn * 96 + j * 32 + fr;
            if (col >= N) continue;
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t row = m0 + wm * 64 + i * 32 + 8 * (e >> 2) + 4 * fh + (e & 3);
                    if (row < M) {
                        if constexpr (kBf16) ((uint16_t*)p.out)[row * N + col] = (uint16_t)f32_to_bf16(acc[i][j][e]);
                        else ((float*)p.out)[row * N + col] = acc[i][j][e];
                    }
                }
        }
    }
}

// FP6 field (sign << 5 | magnitude) of a two's-complement nibble.
__device__ __forceinline__ uint32_t nibble_fp6(uint32_t nib) {
    return nib >= 8u ? 32u | (16u - nib) : nib;
}

// 32 nibbles (16 bytes, channel 2i in the low nibble of byte i) -> 6 dwords of FP6 fields.
__device__ __forceinline__ void nibbles_to_fp6(const uint8_t* src, uint32_t (&w)[6]) {
#pragma unroll
    for (int d = 0; d < 6; ++d) w[d] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const uint32_t field = nibble_fp6((src[j >> 1] >> (4 * (j & 1))) & 15u);
        const int pos = 6 * j;
        w[pos >> 5] |= field << (pos & 31);
        if ((pos & 31) > 26) w[(pos >> 5) + 1] |= field >> (32 - (pos & 31));
    }
}

// ---------------------------------------------------------------- weight prepack
// One 64-thread block per (32-column block, group); lane L covers column L % 32 and
// channel half L / 32 of the group: the B-operand lane of the FP6 MFMA.
__global__ __launch_bounds__(64) void prepack_wgt_kernel(int N, int K, int ncb,
                                                         const uint8_t* __restrict__ wcodes,
                                                         const float* __restrict__ wscales,
                                                         uint8_t* __restrict__ out) {
    const int G = K >> 6;
    const int g = blockIdx.x / ncb, cb = blockIdx.x % ncb;
    const int L = threadIdx.x, col = L & 31, half = L >> 5;
    const int n = cb * 32 + col;
    const bool valid = n < N;
    uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    if (valid) nibbles_to_fp6(wcodes + (int64_t)n * (K / 2) + g * 32 + half * 16, w);
    uint8_t* blk = out + wgt_block(n, g, G);
    *reinterpret_cast<uint4*>(blk + frag_dword(L, 0)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(blk + frag_dword(L, 4)) = make_uint2(w[4], w[5]);
    const float w64 = valid ? wscales[(int64_t)n * G + g] * 64.0f : 0.0f;
    *reinterpret_cast<uint2*>(blk + kFrag + 8 * L) = wgt_scale_operand(w64, L);
}

// ---------------------------------------------------------------- activation pack
// Nibble codes + fp32 scales (the svdq_quantize_act layout) -> packed activations.  One
// 64-thread block per (32-row block, group); rows >= M become zero.
__global__ __launch_bounds__(64) void pack_act_kernel(int64_t M, int K, int64_t nrb,
                                                      const uint8_t* __restrict__ acodes,
                                                      const float* __restrict__ ascales,
                                                      uint8_t* __restrict__ out) {
    const int G = K >> 6;
    const int64_t rb = (int64_t)blockIdx.x % nrb;
    const int g = (int)((int64_t)blockIdx.x / nrb);
    const int L = threadIdx.x, r = L & 31, half = L >> 5;
    const int64_t m = rb * 32 + r;
    const bool valid = m < M;
    uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    if (valid) nibbles_to_fp6(acodes + m * (K / 2) + g * 32 + half * 16, w);
    uint8_t* blk = out + act_block(m, g, G);
    *reinterpret_cast<uint4*>(blk + frag_dword(L, 0)) = make_uint4(w[0], w[1], w[2], w[3]);
    *reinterpret_cast<uint2*>(blk + frag_dword(L, 4)) = make_uint2(w[4], w[5]);
    if (half == 0)
        *reinterpret_cast<uint2*>(blk + kFrag + 8 * r) = act_scale_pair(valid ? ascales[m * G + g] : 0.0f);
}

}  // namespace

void launch_prepack_wgt(int N, int K, const void* wcodes, const void* wscales, void* out,
                        hipStream_t st) {
    const int G = K / 64;
    const int ncb = (N + kBN - 1) / kBN * kCB;
    hipLaunchKernelGGL(prepack_wgt_kernel, dim3(G * ncb), dim3(64), 0, st, N, K, ncb,
                       (const uint8_t*)wcodes, (const float*)wscales, (uint8_t*)out);
}

void launch_pack_act(int64_t M, int K, const void* acodes, const void* ascales, void* out,
                     hipStream_t st) {
    const int G = K / 64;
    const int64_t nrb = (M + kBM - 1) / kBM * kRB;
    hipLaunchKernelGGL(pack_act_kernel, dim3((unsigned)(G * nrb)), dim3(64), 0, st, M, K, nrb,
                       (const uint8_t*)acodes, (const float*)ascales, (uint8_t*)out);
}

template <bool kBf16, bool kGelu, bool kNext = false>
bool set_lds_attr() {
    return hipFuncSetAttribute((const void*)gemm_w4a4_fp6_kernel<kBf16, kGelu, kNext>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, kSmemBytes) == hipSuccess;
}

// The K-split tiles t >= nfull: out = sum over splits s = 0, 1, ... of the partial tiles in
// workspace slots (t - nfull) * nsplit + s, added in that order (bit-reproducible).  Block b
// takes 256 of the 12288 16-byte pieces of tile nfull + b / 48; a piece holds four rows of
// one column (the accumulators' order, see the kernel's K-split store).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ ws,
                                                         float* __restrict__ out, int64_t M, int N,
                                                         int nfull, int nsplit) {
    const int num_m = (int)((M + kBM - 1) / kBM), num_n = (N + kBN - 1) / kBN;
    const int u = blockIdx.x / 48;
    int pid_m, pid_n;
    tile_of(nfull + u, pid_m, pid_n, num_m, num_n);
    const int f = (blockIdx.x % 48) * 256 + threadIdx.x;   // piece in the tile
    const int lane = f & 63, e4 = (f >> 6) & 3, j = (f >> 8) % 3, i = (f / 768) & 1, wave = f / 1536;
    const float* src = ws + (int64_t)u * nsplit * (kBM * kBN) + 4 * f;
    f32x4 v = *reinterpret_cast<const f32x4*>(src);
    for (int s = 1; s < nsplit; ++s) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(src + (int64_t)s * (kBM * kBN));
        v = f32x4{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
    }
    const int col = pid_n * kBN + (wave & 1) * 96 + j * 32 + (lane & 31);
    const int64_t row0 = (int64_t)pid_m * kBM + (wave >> 1) * 64 + i * 32 + 8 * e4 + 4 * (lane >> 5);
    if (col < N) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (row0 + k < M) out[(row0 + k) * N + col] = v[k];
    }
}

// The next layer's lora_act from the fused epilogue's per-tile partial sums: lora[m, j] =
// bf16(sum over the column tiles t of ws[t][m][j]), rounded once to nearest even, in a fixed
// order: the tiles are cut into kLoraChunks consecutive runs, each run summed in order by
// its own thread, then the run sums added in order.  A block holds 32 items (a row's four
// consecutive ranks) x kLoraChunks runs.
constexpr int kLoraChunks = 8;
__global__ __launch_bounds__(256) void sum_lora_kernel(const float* __restrict__ ws,
                                                       uint16_t* __restrict__ lora, int64_t M,
                                                       int64_t Mpad, int R2, int ntn) {
    __shared__ f32x4 part[kLoraChunks][32];
    const int it = threadIdx.x & 31, c = threadIdx.x >> 5;
    const int64_t idx = (int64_t)blockIdx.x * 32 + it;   // (m, 4 ranks)
    const int q = R2 / 4;
    const bool ok = idx < M * q;
    const int64_t m = ok ? idx / q : 0;
    const int j = ok ? 4 * (int)(idx % q) : 0;
    const int run = (ntn + kLoraChunks - 1) / kLoraChunks;
    const int t0 = c * run, t1 = min(ntn, t0 + run);
    const float* src = ws + m * R2 + j;
    const int64_t stride = Mpad * R2;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (ok && t0 < t1) {
        v = *reinterpret_cast<const f32x4*>(src + t0 * stride);
        for (int t = t0 + 1; t < t1; ++t) {
            const f32x4 w = *reinterpret_cast<const f32x4*>(src + t * stride);
            v = f32x4{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
        }
    }
    part[c][it] = v;
    __syncthreads();
    if (c != 0 || !ok) return;
    for (int k = 1; k < kLoraChunks; ++k)
        if (k * run < ntn) {
            const f32x4 w = part[k][it];
            v = f32x4{v[0] + w[0], v[1] + w[1], v[2] + w[2], v[3] + w[3]};
        }
    const uint32_t lo = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    const uint32_t hi = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(lora + m * R2 + j) = make_uint2(lo, hi);
}

int cu_count() {
    static int n[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (n[dev] == 0) {
        int c = 0;
        n[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0 ? c : 256;
    }
    return n[dev];
}

bool gemm_w4a4_fp6_init() {
    static int ok = -1;
    if (ok < 0)
        ok = set_lds_attr<false, false>() && set_lds_attr<false, true>() &&
             set_lds_attr<true, false>() && set_lds_attr<true, true>() &&
             set_lds_attr<true, false, true>() && set_lds_attr<true, true, true>();
    return ok == 1;
}

// Workspace of the K split: nsplit partial tiles for each of the `last` tiles of the last
// round.  One tile per CU and round: when that round would be at most a quarter full, its
// tiles are split over K so that it fills the GPU (fp32 output without GELU only), up to 8
// splits of at least two groups, as many as kSplitWorkspaceMax and the caller's workspace
// hold; with fewer than two splits there is no split.
struct SplitPlan {
    int nfull, nsplit, gsplit;
};
SplitPlan split_plan(int64_t M, int N, int K, int act_fn, int out_bf16, int64_t ws_bytes) {
    const int num_m = (int)((M + kBM - 1) / kBM), num_n = (N + kBN - 1) / kBN;
    const int nt = num_m * num_n, G = K >> 6;
    SplitPlan sp{nt, 1, G};
    const int ncu = cu_count();
    const int last = nt % ncu;
    if (out_bf16 || act_fn != 0 || nt <= ncu || last == 0 || 4 * last > ncu || G < 16) return sp;
    const int64_t tile_bytes = (int64_t)kBM * kBN * 4;
    const int64_t cap = std::min<int64_t>(ws_bytes, kSplitWorkspaceMax) / (tile_bytes * last);
    int want = (int)std::min<int64_t>(std::min(8, ncu / last), cap);
    if (want < 2) return sp;
    sp.gsplit = (G + want - 1) / want;
    sp.nsplit = (G + sp.gsplit - 1) / sp.gsplit;
    sp.nfull = nt - last;
    return sp;
}

int64_t split_workspace_bytes(int64_t M, int N, int K, int act_fn, int out_bf16) {
    const SplitPlan sp = split_plan(M, N, K, act_fn, out_bf16, kSplitWorkspaceMax);
    if (sp.nsplit < 2) return 0;
    const int num_m = (int)((M + kBM - 1) / kBM), num_n = (N + kBN - 1) / kBN;
    return (int64_t)(num_m * num_n - sp.nfull) * sp.nsplit * kBM * kBN * 4;
}

int64_t quantize_next_workspace_bytes(int64_t M, int N, int next_r) {
    const int64_t Mpad = (M + kBM - 1) / kBM * kBM;
    return (int64_t)((N + kBN - 1) / kBN) * Mpad * next_r * 4;
}

void launch_gemm_w4a4_fp6(const PackedGemmArgs& a, hipStream_t st) {
    const int num_m = (int)((a.M + kBM - 1) / kBM), num_n = (a.N + kBN - 1) / kBN;
    const int nt = num_m * num_n;
    PackedGemmArgs b = a;
    const int esz = a.out_bf16 ? 2 : 4;
    b.vec_store = ((int64_t)a.N * esz) % 16 == 0 && (reinterpret_cast<uintptr_t>(a.out) % 16) == 0;
    const SplitPlan sp = a.quantize_next || a.split_ws == nullptr
                             ? SplitPlan{nt, 1, a.K >> 6}
                             : split_plan(a.M, a.N, a.K, a.act_fn, a.out_bf16, a.split_ws_bytes);
    b.nfull = sp.nfull;
    b.nsplit = sp.nsplit;
    b.gsplit = sp.gsplit;
    const dim3 grid(b.nfull + (nt - b.nfull) * b.nsplit), block(kThreads);
    if (a.quantize_next) {   // the next layer's low-rank sums: per-tile partials, then summed
        if (a.act_fn == 1) hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<true, true, true>), grid, block, kSmemBytes, st, b);
        else hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<true, false, true>), grid, block, kSmemBytes, st, b);
        if (a.next_r > 0) {
            const int64_t n = a.M * (a.next_r / 4);
            hipLaunchKernelGGL(sum_lora_kernel, dim3((unsigned)((n + 31) / 32)), dim3(256), 0, st,
                               (const float*)a.lora_work, (uint16_t*)a.out, a.M, (int64_t)num_m * kBM,
                               a.next_r, num_n);
        }
        return;
    }
    if (a.out_bf16) {
        if (a.act_fn == 1) hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<true, true>), grid, block, kSmemBytes, st, b);
        else hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<true, false>), grid, block, kSmemBytes, st, b);
    } else {
        if (a.act_fn == 1) hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<false, true>), grid, block, kSmemBytes, st, b);
        else hipLaunchKernelGGL((gemm_w4a4_fp6_kernel<false, false>), grid, block, kSmemBytes, st, b);
    }
    if (b.nsplit > 1)
        hipLaunchKernelGGL(sum_splits_kernel, dim3(48 * (nt - b.nfull)), dim3(256), 0, st,
                           (const float*)a.split_ws, (float*)a.out, a.M, a.N, b.nfull, b.nsplit);
}

}  // namespace svdq

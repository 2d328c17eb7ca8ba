// awq.hip -- AWQ W4A16 GEMV / skinny GEMM for modulation layers (page "Diffusers Natively
// Integrates Nunchaku Lite ...", third paragraph: sensitive or bandwidth-bound modulation
// layers keep 16-bit activations with 4-bit weights; kernel family awq_w4a16, page "Hugging
// Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 3).
//
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] (q[n,k] - z[n,g]) + b[n]
//
// The layer streams 0.56 bytes per weight and does 2M flops with it, so it is bound by HBM
// as long as turning codes into numbers costs little VALU time.  A 4-bit code q becomes the
// exact bf16 value 128 + q by putting the byte 0x43 above it (bf16 0x4300 | q = 128 + q),
// which one v_perm does for two codes, and a bf16 MFMA forms the dot products:
//   sum_{k in g} x (q - z) = sum_{k in g} x (128 + q) - (128 + z) sum_{k in g} x,
// with the per-group sums of x computed once per block.  Products of two bf16 values are
// exact in fp32 and the MFMA accumulates in fp32.
//
// Fast kernel (M <= 4, K a multiple of 512 up to 4096): one workgroup per CU, each owning
// an equal run of output columns (weight rows), so every CU streams the same number of
// bytes.  Every wave copies its share of x, the scales and zeros, and its K slice (4 groups
// = 128 bytes of every weight row of the run) into LDS with global_load_lds_dwordx4, two
// half tiles of codes ahead of the tile it computes; every code copy reads 8 rows x 128
// contiguous bytes.  Within each 8-row x 128-byte block the 16-byte chunks are stored
// XOR-swizzled by row, so that the MFMA-operand reads below are free of bank conflicts.
// Wave w then runs v_mfma_f32_16x16x32_bf16 over its slice, 16 columns at a time, as soon
// as the copies of each 16 columns have landed; lane L holds column L % 16 and codes
// 16 (L / 16) .. + 15 of each group, x comes from LDS as the A operand (lanes 0-15 of the
// result hold rows 0-3).  The slices are added through LDS in a fixed order.
//
// Reference kernel (any M and K): one wave per output row, fp32 FMAs.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

// ------------------------------------------------------------------------- fast kernel
constexpr int kAwqRows = 4;        // token rows (M) the fast kernel takes
constexpr int kAwqSliceGroups = 4; // groups per wave: 128 bytes of each weight row
constexpr int kAwqMaxTiles = 8;    // 16-column tiles per workgroup
constexpr int kAwqLds = 160 * 1024;

// s_waitcnt vmcnt(n), lgkmcnt(0)
template <int n>
__device__ __forceinline__ void awq_wait_vm() {
    __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
}
__device__ __forceinline__ void awq_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
typedef __attribute__((address_space(3))) uint8_t awq_lds_u8;
__device__ __forceinline__ uint32_t awq_lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(awq_lds_u8*)p);
}
// Global -> LDS copy of 1 KiB: lane l moves the 16 bytes at gaddr (its own address) to LDS
// byte lds + 16 l.  Through asm, so that the compiler does not drain the copies before LDS
// reads of other buffers; completion is tracked with awq_wait_vm.  The s_nop is the wait
// state an LDS DMA needs after an SALU write of M0.
__device__ __forceinline__ void awq_dma(const void* gaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(gaddr), "s"(lds) : "memory");
}

// Per-wave LDS region (wave w = K slice w, groups 4 w .. 4 w + 3), bytes:
//   codes  [H = cols / 8 halves][8 rows][128 B]   16-byte chunks XOR-swizzled by row
//   x      [ceil(M / 2) KiB]  rows m of the slice, 512 B each
//   scales [2 (scale, zero)][cols][16 B] (the 16-byte piece holding the slice's 4 groups)
//          + 320 B: the x sums [4 groups][4 rows] fp32, and in wave 0 the bias of the
//          workgroup's columns (<= 128 bf16); the scale reads of a partial last tile (at
//          most 240 B past the copied pieces) may land there
// Everything a wave reads is copied by that wave, so waves run without barriers until the
// slices are added; each keeps kAwqAhead half tiles of codes in flight (below).
struct AwqRegion {
    int halves, xkb, sbytes;
    __host__ __device__ AwqRegion(int64_t M, int cols)
        : halves((cols + 7) / 8), xkb((int)((M + 1) / 2)), sbytes((2 * cols + 63) / 64 * 1024 + 320) {}
    __host__ __device__ int bytes() const { return (halves + xkb) * 1024 + sbytes; }
};

__host__ inline size_t awq_lds_bytes(int64_t M, int K, int cols) {
    return (size_t)(K / 64 / kAwqSliceGroups) * AwqRegion(M, cols).bytes();
}

// Half tiles of codes in flight per wave: a tile reads two, so at least 2; the tile after
// the current one goes out as soon as the current tile's codes are in registers.  Fewer in
// flight per wave measured faster (9.3 us at 2, 9.5 at 3, 9.7 at 4 on the modulation
// layer, M = 2, K = 3072, N = 18432); the twelve waves of a CU still keep ~24 in flight.
constexpr int kAwqAhead = 2;
static_assert(kAwqAhead >= 2, "a tile reads two half tiles");

__device__ __forceinline__ void awq_wait_vm_rt(int n) {   // n in [0, 16]
    switch (n) {
        case 0: awq_wait_vm<0>(); break;   case 1: awq_wait_vm<1>(); break;
        case 2: awq_wait_vm<2>(); break;   case 3: awq_wait_vm<3>(); break;
        case 4: awq_wait_vm<4>(); break;   case 5: awq_wait_vm<5>(); break;
        case 6: awq_wait_vm<6>(); break;   case 7: awq_wait_vm<7>(); break;
        default: awq_wait_vm<8>(); break;
    }
}

__device__ __forceinline__ float quad_sum(float v) {   // sum over lanes 4 i .. 4 i + 3
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
    return v;
}
// Sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (the four 16-lane rows), in every lane.
__device__ __forceinline__ float rows_sum(float v) {
    const uint32_t u = __float_as_uint(v);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);   // rows (0,1) and (2,3)
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const uint32_t us = __float_as_uint(s);
    const auto b = __builtin_amdgcn_permlane32_swap(us, us, false, false);  // halves
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// kW = K / 256 waves, one K slice each.
template <int kW>
__global__ __launch_bounds__(kW * 64) void awq_gemv_lds_kernel(AwqArgs p, int cols) {
    extern __shared__ __align__(16) uint8_t smem[];
    constexpr int kG = kW * kAwqSliceGroups, kK = kW * 256;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int N = p.N, M = (int)p.M;
    const int c0 = blockIdx.x * cols;
    const int c1 = min(N, c0 + cols);   // this workgroup's columns [c0, c1)
    const int tiles = (cols + 15) / 16;
    const AwqRegion reg(M, cols);
    const int H = reg.halves;
    uint8_t* codes = smem + (size_t)w * reg.bytes();
    uint8_t* xw = codes + H * 1024;
    uint8_t* scw = xw + reg.xkb * 1024;
    float* gsl = reinterpret_cast<float*>(scw + reg.sbytes - 320);   // [4 groups][4 rows]
    // bias of the workgroup's columns, copied by wave 0 when 16-byte aligned with N % 8 == 0
    // (a plain load at the end otherwise: no plain global load may sit among the copies, the
    // compiler would wait for it before each one)
    const bool bias_dma = p.bias != nullptr && (reinterpret_cast<uintptr_t>(p.bias) & 15) == 0 && N % 8 == 0;
    const uint16_t* bias_lds = reinterpret_cast<const uint16_t*>(smem + reg.sbytes - 256 + (size_t)(H + reg.xkb) * 1024);

    // ---- copies: the bias (wave 0), x slice, scales and zeros, then the first code halves
    if (w == 0 && bias_dma && lane < (c1 - c0) / 8)
        awq_dma((const uint8_t*)p.bias + (size_t)(c0 + 8 * lane) * 2, awq_lds_addr(bias_lds + 8 * lane));
    for (int j = 0; j < reg.xkb; ++j) {   // x: lane e -> row e / 32, 16 bytes (e % 32) of the slice
        const int e = 64 * j + lane, row = min(e >> 5, M - 1);
        awq_dma((const uint8_t*)p.x + ((size_t)row * kK + 256 * w) * 2 + 16 * (e & 31), awq_lds_addr(xw + 1024 * j));
    }
    const int ns = (2 * cols + 63) / 64;
    for (int j = 0; j < ns; ++j) {        // scales then zeros: lane e -> column e % cols
        const int e = 64 * j + lane;
        const int zero = e >= cols, r = e < 2 * cols ? min(c0 + e % cols, c1 - 1) : c0;
        const uint8_t* src = (const uint8_t*)(zero ? p.zeros : p.scales) + (size_t)r * kG * 2 + 16 * (w >> 1);
        awq_dma(src, awq_lds_addr(scw + 1024 * j));
    }
    // codes: copy j covers rows 8 j .. + 7; lane l fetches row l / 8, chunk (l % 8) ^ (l / 8)
    const int cr8 = lane >> 3, csl = lane & 7;
    const uint8_t* qsrc = (const uint8_t*)p.qweight + (size_t)128 * w + 16 * (csl ^ cr8);
    auto copy_half = [&](int j) {
        const int r = min(c0 + 8 * j + cr8, c1 - 1);
        awq_dma(qsrc + (size_t)r * (kK / 2), awq_lds_addr(codes + 1024 * j));
    };
    const int first = min(H, kAwqAhead);
    for (int j = 0; j < first; ++j) copy_half(j);
    awq_wait_vm_rt(first);   // x, scales and zeros have landed

    // ---- per-group sums of x over the slice: lane -> row lane / 16, group (lane / 4) % 4,
    // 16 channels (lane % 4), added over the quad
    {
        const int m = lane >> 4, i = (lane >> 2) & 3, part = lane & 3;
        float sum = 0.0f;
        if (m < M) {
            const uint8_t* src = xw + m * 512 + (64 * i + 16 * part) * 2;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * h);
                const uint32_t wq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int t = 0; t < 4; ++t) sum += bf16_to_f32(wq[t] & 0xFFFFu) + bf16_to_f32(wq[t] >> 16);
            }
        }
        sum = quad_sum(sum);
        if (part == 0) gsl[i * 4 + m] = sum;
    }

    // ---- A operands, block diagonal: MFMA row r = 4 gi + m holds x row m on the channels of
    // group gi (zero elsewhere), so one accumulator collects the four groups apart; lane L
    // supplies row L % 16, channels 16 kq + 8 j .. +7 of the group (kq = L / 16), reordered
    // even channels first to match the codes below
    const int col = lane & 15, kq = lane >> 4;
    uint4 xa[kAwqSliceGroups][2];
    {
        const int am = col & 3, agi = col >> 2;
        const uint8_t* xr = xw + min(am, M - 1) * 512 + (64 * agi + 16 * kq) * 2;
        uint4 xv[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 v = *reinterpret_cast<const uint4*>(xr + 16 * j);
            uint4 o;
            o.x = __builtin_amdgcn_perm(v.y, v.x, 0x05040100u);   // x0 x2
            o.y = __builtin_amdgcn_perm(v.w, v.z, 0x05040100u);   // x4 x6
            o.z = __builtin_amdgcn_perm(v.y, v.x, 0x07060302u);   // x1 x3
            o.w = __builtin_amdgcn_perm(v.w, v.z, 0x07060302u);   // x5 x7
            xv[j] = o;
        }
#pragma unroll
        for (int gi = 0; gi < kAwqSliceGroups; ++gi)
#pragma unroll
            for (int j = 0; j < 2; ++j) xa[gi][j] = gi == agi ? xv[j] : make_uint4(0u, 0u, 0u, 0u);
    }
    // this lane's result rows: group kq, rows 0-3 of column col; their x sums
    const float4 gsv = *reinterpret_cast<const float4*>(gsl + 4 * kq);

    // ---- tiles of 16 columns, each as soon as its copies have landed
    const int hr = col >> 3, r8 = col & 7;
    const int soff = 2 * (4 * (w & 1) + kq);   // this lane's group in the 16-byte scale piece
    for (int t = 0; t < tiles; ++t) {
        awq_wait_vm_rt(max(0, min(H - 2 * t - 2, kAwqAhead - 2)));
        const float sc = bf16_to_f32(*reinterpret_cast<const uint16_t*>(scw + 16 * (16 * t + col) + soff));
        const float zz = 128.0f + bf16_to_f32(*reinterpret_cast<const uint16_t*>(scw + 16 * (cols + 16 * t + col) + soff));
        const uint8_t* blk = codes + (size_t)(2 * t + hr) * 1024 + 128 * r8 + 8 * (kq & 1);
        uint2 cv[kAwqSliceGroups];
#pragma unroll
        for (int gi = 0; gi < kAwqSliceGroups; ++gi)
            cv[gi] = *reinterpret_cast<const uint2*>(blk + 16 * ((2 * gi + (kq >> 1)) ^ r8));
        // the next copies go out as soon as this tile's codes are in registers
        if (2 * t + kAwqAhead < H) copy_half(2 * t + kAwqAhead);
        if (2 * t + kAwqAhead + 1 < H) copy_half(2 * t + kAwqAhead + 1);
        f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int gi = 0; gi < kAwqSliceGroups; ++gi) {
            const uint32_t cw[2] = {cv[gi].x, cv[gi].y};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                // codes 8 j .. 8 j + 7 of this lane's 16 (low nibble first): even codes in the
                // bytes of e, odd ones in the bytes of o; each becomes the bf16 0x43 | code
                const uint32_t e = cw[j] & 0x0F0F0F0Fu, o = (cw[j] >> 4) & 0x0F0F0F0Fu;
                uint4 bq;
                bq.x = __builtin_amdgcn_perm(0x43434343u, e, 0x04010400u);
                bq.y = __builtin_amdgcn_perm(0x43434343u, e, 0x04030402u);
                bq.z = __builtin_amdgcn_perm(0x43434343u, o, 0x04010400u);
                bq.w = __builtin_amdgcn_perm(0x43434343u, o, 0x04030402u);
                r = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[gi][j]), as_bf16x8(bq), r, 0, 0, 0);
            }
        }
        // r[m] = sum over group kq of x[m,k] (128 + q[n,k]); scale, add over the groups
        const float v[kAwqRows] = {sc * fmaf(-zz, gsv.x, r[0]), sc * fmaf(-zz, gsv.y, r[1]),
                                   sc * fmaf(-zz, gsv.z, r[2]), sc * fmaf(-zz, gsv.w, r[3])};
        float* red = reinterpret_cast<float*>(codes + (size_t)t * 2048);   // [rows][16], tile t's first codes
#pragma unroll
        for (int m = 0; m < kAwqRows; ++m) {
            if (m < M) {
                const float tot = rows_sum(v[m]);
                if (kq == 0) red[m * 16 + col] = tot;
            }
        }
    }

    // ---- add the slices in wave order
    __syncthreads();
    const int i = threadIdx.x;
    if (i < tiles * 16 && c0 + i < c1) {
        const int n = c0 + i, t = i >> 4, c = i & 15;
        float bv = 0.0f;
        if (bias_dma) bv = bf16_to_f32(bias_lds[i]);
        else if (p.bias != nullptr) bv = bf16_to_f32(((const uint16_t*)p.bias)[n]);
        for (int m = 0; m < M; ++m) {
            float part[kW];
#pragma unroll
            for (int sl = 0; sl < kW; ++sl)
                part[sl] = reinterpret_cast<const float*>(smem + (size_t)sl * reg.bytes() + (size_t)t * 2048)[m * 16 + c];
            float v = 0.0f;
#pragma unroll
            for (int sl = 0; sl < kW; ++sl) v += part[sl];
            v += bv;
            const int64_t idx = (int64_t)m * N + n;
            if (p.out_bf16) ((uint16_t*)p.out)[idx] = (uint16_t)f32_to_bf16(v);
            else ((float*)p.out)[idx] = v;
        }
    }
}

// --------------------------------------------------------------------- reference kernel
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

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Columns per workgroup for the fast kernel: an equal share per CU (multiple of 8), fewer
// when the LDS regions do not fit; 0 when the fast kernel does not apply.
int awq_fast_cols(const AwqArgs& a) {
    const int G = a.K / 64;
    if (a.M < 1 || a.M > kAwqRows || G % 8 != 0 || G > 64) return 0;
    // the copies move 16-byte pieces of x, the codes, the scales and the zeros
    if (((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.qweight) |
          reinterpret_cast<uintptr_t>(a.scales) | reinterpret_cast<uintptr_t>(a.zeros)) & 15) != 0)
        return 0;
    const int cus = cu_count();
    int cols = (a.N + cus - 1) / cus;
    cols = (cols + 7) / 8 * 8;
    if (cols > 16 * kAwqMaxTiles) cols = 16 * kAwqMaxTiles;
    while (cols > 8 && awq_lds_bytes(a.M, a.K, cols) > (size_t)kAwqLds) cols -= 8;
    return awq_lds_bytes(a.M, a.K, cols) <= (size_t)kAwqLds ? cols : 0;
}

template <int kW>
void launch_lds(const AwqArgs& a, int cols, hipStream_t st) {
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void*)awq_gemv_lds_kernel<kW>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kAwqLds);
        attr = true;
    }
    hipLaunchKernelGGL(awq_gemv_lds_kernel<kW>, dim3((unsigned)((a.N + cols - 1) / cols)), dim3(kW * 64),
                       awq_lds_bytes(a.M, a.K, cols), st, a, cols);
}

}  // namespace

void launch_awq_gemv(const AwqArgs& a, hipStream_t st) {
    const int cols = awq_fast_cols(a);
    if (cols > 0) {
        switch (a.K / 256) {
            case 2: return launch_lds<2>(a, cols, st);
            case 4: return launch_lds<4>(a, cols, st);
            case 6: return launch_lds<6>(a, cols, st);
            case 8: return launch_lds<8>(a, cols, st);
            case 10: return launch_lds<10>(a, cols, st);
            case 12: return launch_lds<12>(a, cols, st);
            case 14: return launch_lds<14>(a, cols, st);
            case 16: return launch_lds<16>(a, cols, st);
            default: break;
        }
    }
    dim3 grid((unsigned)((a.N + kWavesPerBlock - 1) / kWavesPerBlock));
    hipLaunchKernelGGL(awq_gemv_v0_kernel, grid, dim3(kWavesPerBlock * 64), 0, st, a);
}

}  // namespace svdq

// weights.hip -- the offline weight side of SVDQuant on gfx950 (page "Hugging Face 把 Nunchaku
// 4-bit Diffusion 接到 Diffusers", 技术细节 1, "SVDQuant 的核心思路" and the quantize-your-own-
// model walk-through; page "Diffusers integra Nunchaku ...", the section on quantizing a model
// with diffuse-compressor): calibration absmax, per-channel smoothing factors, and the 4-bit
// residual of the smoothed weight once the 16-bit low-rank branch is taken out.  All three are
// HBM-bound elementwise or column reductions; the residual's low-rank product runs in fp64 so
// that the residual, and with it every code and scale, is the exact result of its definition.
#include "common.hpp"
#include "launch.hpp"
#include "quant_lane.hpp"

namespace svdq {
namespace {

constexpr int kColThreads = 256, kColRows = 32;   // column pieces per block, rows per block
constexpr int kCalPieces = 64, kCalGroups = 4, kCalRows = 16;   // calibration block shape

// out[c] = max(out[c], max |x[r, c]|) over bf16 x [M, K].  A block covers 64 pieces of 8
// columns and 64 rows: its four waves take 16 rows each (16 loads in flight per lane), the
// LDS combines the four, and one atomic per column leaves the block.  |x| as fp32 bits:
// non-negative floats order like their bit patterns (a NaN ranks above every number, so it
// survives the max as it does in the definition's max).
__global__ __launch_bounds__(kCalPieces * kCalGroups) void col_absmax_bf16_kernel(
    const uint16_t* __restrict__ x, int64_t M, int K, unsigned* __restrict__ out) {
    __shared__ uint32_t part[kCalGroups][8][kCalPieces];
    const int pc = threadIdx.x & (kCalPieces - 1), grp = threadIdx.x / kCalPieces;
    const int c8 = blockIdx.x * kCalPieces + pc;
    const bool ok = 8 * c8 < K;
    const int64_t r0 = (int64_t)blockIdx.y * (kCalRows * kCalGroups) + grp * kCalRows;
    uint32_t m[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < kCalRows; ++i) {
        const int64_t r = r0 + i;
        if (ok && r < M) {
            const uint4 v = *reinterpret_cast<const uint4*>(x + r * K + 8 * c8);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                m[2 * j] = max(m[2 * j], (w[j] & 0x7FFFu) << 16);
                m[2 * j + 1] = max(m[2 * j + 1], w[j] & 0x7FFF0000u);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part[grp][j][pc] = m[j];
    __syncthreads();
    if (grp == 0 && ok) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t v = part[0][j][pc];
#pragma unroll
            for (int q = 1; q < kCalGroups; ++q) v = max(v, part[q][j][pc]);
            atomicMax(out + 8 * c8 + j, v);
        }
    }
}

// the same over fp32 w [N, K], 4 columns per thread
__global__ __launch_bounds__(kColThreads) void col_absmax_f32_kernel(const float* __restrict__ w,
                                                                     int64_t N, int K,
                                                                     unsigned* __restrict__ out) {
    const int c4 = blockIdx.x * kColThreads + threadIdx.x;
    if (4 * c4 >= K) return;
    const int64_t r0 = (int64_t)blockIdx.y * kColRows, r1 = min(N, r0 + kColRows);
    uint32_t m[4] = {0u, 0u, 0u, 0u};
#pragma unroll 8
    for (int64_t r = r0; r < r1; ++r) {
        const uint4 v = *reinterpret_cast<const uint4*>(w + r * K + 4 * c4);
        m[0] = max(m[0], v.x & 0x7FFFFFFFu);
        m[1] = max(m[1], v.y & 0x7FFFFFFFu);
        m[2] = max(m[2], v.z & 0x7FFFFFFFu);
        m[3] = max(m[3], v.w & 0x7FFFFFFFu);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicMax(out + 4 * c4 + i, m[i]);
}

__global__ __launch_bounds__(256) void fill_zero_u32_kernel(unsigned* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Smoothing factor of channel k, migrating activation outliers into the weight (技术细节 1
// step 1): lambda = sqrt(cx / cw) in binary64 (1 where it is not a positive finite number or
// either maximum is 0), stored as smooth_inv = fp32(1 / lambda).  Each operation is one
// correctly rounded binary64 operation, so the result is a function of (cx, cw) alone.
__global__ __launch_bounds__(256) void smooth_factor_kernel(const float* __restrict__ cx,
                                                            const float* __restrict__ cw, int K,
                                                            float* __restrict__ smooth_inv) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= K) return;
    const double a = cx[k], b = cw[k];
    double lam = __builtin_sqrt(a / b);
    if (!__builtin_isfinite(lam) || lam == 0.0 || a == 0.0 || b == 0.0) lam = 1.0;
    smooth_inv[k] = (float)(1.0 / lam);
}

// The 4-bit residual of one layer (技术细节 1 steps 2 and 3).  With lam_k = 1 / smooth_inv[k]
// (binary64), the smoothed weight is w_hat = w lam_k; the low-rank branch carries
// (l2 l1)[n, k] lam_k (l1 absorbs smooth_inv, so un-smoothing it gives the branch's share of
// w_hat); the residual is R = fp32(w_hat - (l2 l1) lam).  (l2 l1)[n, k] sums r products of
// two bf16 values.  Each product is exact in binary64: a 16-bit integer times 2^e_j.  Their
// sum, and every partial sum, is then an integer multiple of 2^(min e_j) below
// r 2^16 2^(max e_j), exact in binary64's 53 bits while max e_j - min e_j <= 37 - ceil(log2 r)
// (32 at rank 32, 30 at rank 128); within that no summation order changes it.  Thread t:
// row t / (K / 32), channels 32 (t % (K / 32)) .. + 31; the lanes t, t ^ 1 share a 64-group.
struct ResidualArgs {
    const float* w;
    const float* smooth_inv;
    const uint16_t* l1;
    const uint16_t* l2;
    int N, K, r;
    uint8_t* codes;
    void* scales;
    unsigned* gmax;   // NVFP4: the residual's max |R| (fp32 bits), then S_w
};

__device__ __forceinline__ lane::Vals residual32(const ResidualArgs& a, int n, int c0) {
#pragma clang fp contract(off)
    const int K = a.K;
    double p[32];
#pragma unroll
    for (int c = 0; c < 32; ++c) p[c] = 0.0;
    for (int j = 0; j < a.r; ++j) {
        const double u = (double)__uint_as_float((uint32_t)a.l2[(int64_t)n * a.r + j] << 16);
        const uint4* lr = reinterpret_cast<const uint4*>(a.l1 + (int64_t)j * K + c0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint4 v = lr[q];
            const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[8 * q + 2 * i] = __builtin_fma(u, (double)__uint_as_float(wd[i] << 16), p[8 * q + 2 * i]);
                p[8 * q + 2 * i + 1] =
                    __builtin_fma(u, (double)__uint_as_float(wd[i] & 0xFFFF0000u), p[8 * q + 2 * i + 1]);
            }
        }
    }
    lane::Vals keep;
    const float4* wr = reinterpret_cast<const float4*>(a.w + (int64_t)n * K + c0);
    const float4* sr = reinterpret_cast<const float4*>(a.smooth_inv + c0);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const float4 wv = wr[q], sv = sr[q];
        const float wf[4] = {wv.x, wv.y, wv.z, wv.w}, sf[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * q + i;
            const double lam = 1.0 / (double)sf[i];
            const double wh = (double)wf[i] * lam;
            const float rv = a.r > 0 ? (float)(wh - p[c] * lam) : (float)wh;
            if (c & 1) keep.od[c >> 1] = rv;
            else keep.ev[c >> 1] = rv;
        }
    }
    return keep;
}

// INT4: per 64-channel group, the activation rule (s = absmax / 7, q = rne(R / s)).
__global__ __launch_bounds__(256) void residual_int4_kernel(ResidualArgs a) {
    const int hpr = a.K >> 5;   // 32-channel halves per row (even)
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)a.N * hpr) return;   // whole pairs: N * hpr is even
    const int n = (int)(t / hpr), hg = (int)(t - (int64_t)n * hpr);
    const lane::Vals keep = residual32(a, n, 32 * hg);
    lane::Vals v = keep;
    float am = lane::absmax32(v);
    am = fmaxf(am, __shfl_xor(am, 1, 64));   // the group's other half
    const float s = am / 7.0f;
    lane::int4_codes32_exact(v, s, [&] { v = keep; });
    uint32_t d[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t pair = ((uint32_t)(int)v.ev[i] & 15u) | (((uint32_t)(int)v.od[i] & 15u) << 4);
        d[i >> 2] |= pair << (8 * (i & 3));
    }
    *reinterpret_cast<uint4*>(a.codes + (int64_t)n * (a.K / 2) + 16 * hg) = make_uint4(d[0], d[1], d[2], d[3]);
    if ((hg & 1) == 0) reinterpret_cast<float*>(a.scales)[(int64_t)n * (a.K / 64) + (hg >> 1)] = s;
}

// NVFP4, first pass: max |R| over the layer (every lane takes part in the wave's reduction;
// lanes past the end contribute 0), one atomic per wave.
__global__ __launch_bounds__(256) void residual_absmax_kernel(ResidualArgs a) {
    const int hpr = a.K >> 5;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    float am = 0.0f;
    if (t < (int64_t)a.N * hpr) {
        const int n = (int)(t / hpr), hg = (int)(t - (int64_t)n * hpr);
        am = lane::absmax32(residual32(a, n, 32 * hg));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
    if ((threadIdx.x & 63) == 0) atomicMax(a.gmax, __float_as_uint(am));
}

// NVFP4, second pass: per-tensor S_w = fp32(max |R| / 2688) (2688 = 448 * 6, the largest
// E4M3 scale times the largest E2M1 value), then the activation rule per 16-block.
__global__ __launch_bounds__(256) void residual_nvfp4_kernel(ResidualArgs a) {
    const int hpr = a.K >> 5;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)a.N * hpr) return;
    const int n = (int)(t / hpr), hg = (int)(t - (int64_t)n * hpr);
    const float S = __uint_as_float(*a.gmax) / 2688.0f;
    const lane::Vals v = residual32(a, n, 32 * hg);
    uint32_t d[4], sbs;
    lane::nvfp4_codes32(v, S, d, sbs);
    *reinterpret_cast<uint4*>(a.codes + (int64_t)n * (a.K / 2) + 16 * hg) = make_uint4(d[0], d[1], d[2], d[3]);
    *reinterpret_cast<uint16_t*>((uint8_t*)a.scales + (int64_t)n * (a.K / 16) + 2 * hg) = (uint16_t)sbs;
}

__global__ void global_scale_kernel(unsigned* g) {
    const float S = __uint_as_float(*g) / 2688.0f;
    *reinterpret_cast<float*>(g) = S;
}

dim3 col_grid(int64_t rows, int K, int per_thread) {
    const int pieces = K / per_thread;
    return dim3((unsigned)((pieces + kColThreads - 1) / kColThreads), (unsigned)((rows + kColRows - 1) / kColRows));
}

}  // namespace

void launch_calib_absmax(int64_t M, int K, const void* x, float* absmax, hipStream_t st) {
    const dim3 grid((unsigned)((K / 8 + kCalPieces - 1) / kCalPieces),
                    (unsigned)((M + kCalRows * kCalGroups - 1) / (kCalRows * kCalGroups)));
    hipLaunchKernelGGL(col_absmax_bf16_kernel, grid, dim3(kCalPieces * kCalGroups), 0, st,
                       (const uint16_t*)x, M, K, reinterpret_cast<unsigned*>(absmax));
}

void launch_smoothing_factors(int N, int K, const float* w, const float* x_absmax, float* w_absmax,
                              float* smooth_inv, hipStream_t st) {
    hipLaunchKernelGGL(fill_zero_u32_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<unsigned*>(w_absmax), K);
    hipLaunchKernelGGL(col_absmax_f32_kernel, col_grid(N, K, 4), dim3(kColThreads), 0, st, w,
                       (int64_t)N, K, reinterpret_cast<unsigned*>(w_absmax));
    hipLaunchKernelGGL(smooth_factor_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                       x_absmax, (const float*)w_absmax, K, smooth_inv);
}

void launch_quantize_residual(int N, int K, int r, bool nvfp4, const float* w,
                              const float* smooth_inv, const void* l1, const void* l2, void* codes,
                              void* scales, float* global_scale, hipStream_t st) {
    const ResidualArgs a{w, smooth_inv, (const uint16_t*)l1, (const uint16_t*)l2, N, K, r,
                         (uint8_t*)codes, scales, reinterpret_cast<unsigned*>(global_scale)};
    const int64_t threads = (int64_t)N * (K / 32);
    const dim3 grid((unsigned)((threads + 255) / 256));
    if (!nvfp4) {
        hipLaunchKernelGGL(residual_int4_kernel, grid, dim3(256), 0, st, a);
        return;
    }
    hipLaunchKernelGGL(fill_zero_u32_kernel, dim3(1), dim3(256), 0, st, a.gmax, 1);
    hipLaunchKernelGGL(residual_absmax_kernel, grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(residual_nvfp4_kernel, grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL(global_scale_kernel, dim3(1), dim3(1), 0, st, a.gmax);
}

}  // namespace svdq

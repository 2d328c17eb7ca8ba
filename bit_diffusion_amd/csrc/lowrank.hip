// lowrank.hip -- the top-r factorization of the smoothed weight on gfx950: the 16-bit
// low-rank branch of SVDQuant carries the leading singular triplets of W diag(lambda) (page
// "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 1 step 2).  Randomized
// subspace iteration (Halko, Martinsson and Tropp, "Finding structure with randomness",
// 2011, the power-iteration scheme with re-orthonormalization after every product):
//   Y = W_hat Omega, Q = orth(Y); then `iters` times Z = orth(W_hat^T Q), Q = orth(W_hat Z);
//   Z = W_hat^T Q (so B = Q^T W_hat = Z^T); B B^T = Z^T Z = U_B diag(sigma^2) U_B^T;
//   U = Q U_B, V = Z U_B diag(1 / sigma);  l1 = bf16(sqrt(sigma) V^T diag(smooth_inv)),
//   l2 = bf16(U sqrt(sigma)).
// The skinny products are LDS-tiled fp32 kernels; orth is CholeskyQR2 with the Gram matrix
// summed in binary64 and the rows solved against its Cholesky factor in binary64; the small
// symmetric eigenproblem is cyclic Jacobi in binary64 on one workgroup.  Tall matrices are stored with 64 columns (the block width), columns past b zero.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

constexpr int kW = 64;   // stored width of every tall matrix, and the maximum block size b

// Y[n, j] = sum_k W[n, k] lam_k X[k, j] (TRANS = false, rows = N, inner = K) or
// Y[k, j] = lam_k sum_n W[n, k] X[n, j] (TRANS = true, rows = K, inner = N).
// A block computes 64 rows x 64 columns; thread (ty, tx) rows 4 ty .. + 3, columns tx + 16 c.
// The inner dimension is cut into gridDim.y slices of `chunk` (a multiple of 32); slice y
// writes its partial product to Y + y * rows * 64 and sum_slices_kernel adds the slices in
// a fixed order, so the result does not depend on scheduling.
template <bool TRANS>
__global__ __launch_bounds__(256) void skinny_kernel(const float* __restrict__ W,
                                                     const float* __restrict__ smooth_inv, int N,
                                                     int K, const float* __restrict__ X, int chunk,
                                                     float* __restrict__ Y) {
    __shared__ float As[32][kW + 1];   // [inner][row]
    __shared__ float Bs[32][kW];       // [inner][column]
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    const int rows = TRANS ? K : N, inner = TRANS ? N : K;
    const int r0 = blockIdx.x * kW;
    const int ib = blockIdx.y * chunk, ie = min(inner, ib + chunk);
    Y += (int64_t)blockIdx.y * rows * kW;
    float acc[4][4] = {};
    for (int i0 = ib; i0 < ie; i0 += 32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int idx = tid + 256 * e;   // 2048 elements of each tile
            if constexpr (!TRANS) {
                const int rr = idx >> 5, ii = idx & 31;   // W[r0 + rr, i0 + ii] * lam
                const int n = r0 + rr, k = i0 + ii;
                As[ii][rr] = n < N && k < ie ? W[(int64_t)n * K + k] / smooth_inv[k] : 0.0f;
            } else {
                const int ii = idx >> 6, rr = idx & 63;   // W[i0 + ii, r0 + rr]
                const int n = i0 + ii, k = r0 + rr;
                As[ii][rr] = n < ie && k < K ? W[(int64_t)n * K + k] : 0.0f;
            }
            const int bi = idx >> 6, bj = idx & 63;
            Bs[bi][bj] = i0 + bi < ie ? X[(int64_t)(i0 + bi) * kW + bj] : 0.0f;
        }
        __syncthreads();
#pragma unroll 8
        for (int ii = 0; ii < 32; ++ii) {
            float a[4], bv[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) a[q] = As[ii][4 * ty + q];
#pragma unroll
            for (int c = 0; c < 4; ++c) bv[c] = Bs[ii][tx + 16 * c];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[q][c] = fmaf(a[q], bv[c], acc[q][c]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int r = r0 + 4 * ty + q;
        if (r >= rows) continue;
        const float scale = TRANS ? 1.0f / smooth_inv[r] : 1.0f;
#pragma unroll
        for (int c = 0; c < 4; ++c) Y[(int64_t)r * kW + tx + 16 * c] = acc[q][c] * scale;
    }
}

// out[r, j] = sum over the slices s = 0, 1, ... of part[s][r, j], in that order
__global__ __launch_bounds__(256) void sum_slices_kernel(const float* __restrict__ part, int64_t n,
                                                         int slices, float* __restrict__ out) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n) return;
    float s = part[t];
    for (int y = 1; y < slices; ++y) s += part[(int64_t)y * n + t];
    out[t] = s;
}

// part[blk] = X[kGramRows blk .. + kGramRows - 1, :]^T X[...] in binary64 (rows past `rows`
// are zero).  Thread tid owns the entries tid + 256 e, e = 0..15, and runs their sums side by
// side over the rows in order (each product of two fp32 values is exact in binary64).
constexpr int kGramRows = 16;
__global__ __launch_bounds__(256) void gram_partial_kernel(const float* __restrict__ X, int rows,
                                                           double* __restrict__ part) {
    __shared__ float xs[kGramRows][kW];
    const int tid = threadIdx.x;
    const int r0 = blockIdx.x * kGramRows;
#pragma unroll
    for (int e = 0; e < kGramRows * kW / 256; ++e) {
        const int idx = tid + 256 * e, rr = idx >> 6, cc = idx & 63;
        xs[rr][cc] = r0 + rr < rows ? X[(int64_t)(r0 + rr) * kW + cc] : 0.0f;
    }
    __syncthreads();
    double s[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.0;
    const int j = tid & 63;
    for (int r = 0; r < kGramRows; ++r) {
        const double xj = xs[r][j];
#pragma unroll
        for (int e = 0; e < 16; ++e) s[e] += (double)xs[r][(tid >> 6) + 4 * e] * xj;
    }
    double* out = part + (int64_t)blockIdx.x * kW * kW;
#pragma unroll
    for (int e = 0; e < 16; ++e) out[tid + 256 * e] = s[e];
}

// gsum[e] = sum of the partial Gram matrices part[k][e], so that the single-wave kernels
// below read one 64 x 64 matrix.  A block takes 64 entries; its eight waves sum consecutive
// eighths of k in order, and the eighths are added in order (a fixed order).
constexpr int kGramParts = 8;
__global__ __launch_bounds__(64 * kGramParts) void gram_sum_kernel(const double* __restrict__ part, int nblk,
                                                                   double* __restrict__ gsum) {
    __shared__ double qs[kGramParts][64];
    const int q = threadIdx.x >> 6, c = threadIdx.x & 63, e = blockIdx.x * 64 + c;   // grid: kW * kW / 64
    const int len = (nblk + kGramParts - 1) / kGramParts, k0 = q * len, k1 = min(nblk, k0 + len);
    double s = 0.0;
#pragma unroll 4
    for (int k = k0; k < k1; ++k) s += part[(int64_t)k * kW * kW + e];
    qs[q][c] = s;
    __syncthreads();
    if (q == 0) {
        double v = qs[0][c];
#pragma unroll
        for (int i = 1; i < kGramParts; ++i) v += qs[i][c];
        gsum[e] = v;
    }
}

// A summed Gram matrix (64 x 64, b x b used) into LDS, zero outside b x b: threads t < 64
// copy column t.
__device__ void load_gram(const double* g, int b, double (*G)[kW + 1]) {
    const int t = threadIdx.x;
    if (t < kW)
#pragma unroll 8
        for (int i = 0; i < kW; ++i) G[i][t] = i < b && t < b ? g[i * kW + t] : 0.0;
    __syncthreads();
}

// Sum the partial Gram matrices into LDS (b x b used), one wave: lane t keeps column t of
// all 64 rows in registers, so each partial's 64 loads are independent.
__device__ void sum_gram(const double* part, int nblk, int b, double (*G)[kW + 1]) {
    const int t = threadIdx.x;
    double acc[kW];
#pragma unroll
    for (int i = 0; i < kW; ++i) acc[i] = 0.0;
    if (t < b)
        for (int k = 0; k < nblk; ++k) {
            const double* pk = part + (int64_t)k * kW * kW + t;
#pragma unroll
            for (int i = 0; i < kW; ++i) acc[i] += pk[i * kW];
        }
    if (t < kW)
#pragma unroll
        for (int i = 0; i < kW; ++i) G[i][t] = i < b ? acc[i] : 0.0;
    __syncthreads();
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)u, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// CholeskyQR step, factorization: G = L L^T.  Writes lt = L^T (64 x 64, binary64, zero
// outside b x b) and invd[i] = 1 / L[i][i] (0 where the pivot is not positive: a
// rank-deficient block, whose column then drops out).  One wave of 64 lanes.
__global__ __launch_bounds__(64) void chol_kernel(const double* __restrict__ part, int nblk, int b,
                                                  double* __restrict__ lt, double* __restrict__ invd) {
    __shared__ double G[kW][kW + 1];   // padded: column walks stay conflict-free
    __shared__ double L[kW][kW + 1];   // padded: column walks stay conflict-free
    const int t = threadIdx.x;
    sum_gram(part, nblk, b, G);
    for (int i = 0; i < kW; ++i) L[i][t] = 0.0;
    __syncthreads();
    for (int j = 0; j < b; ++j) {
        // lanes i >= j: the column below the pivot (the pivot itself on lane j)
        double s = G[t < kW ? t : 0][j];
#pragma unroll 8
        for (int k = 0; k < j; ++k) s -= L[t][k] * L[j][k];   // loads run ahead, sums in order
        __syncthreads();
        if (t == j) L[j][j] = s > 0.0 ? __builtin_sqrt(s) : 0.0;
        __syncthreads();
        if (t > j && t < b) L[t][j] = L[j][j] > 0.0 ? s / L[j][j] : 0.0;
        __syncthreads();
    }
    for (int k = 0; k < kW; ++k) lt[k * kW + t] = L[t][k];   // lt[k][t] = L[t][k]
    invd[t] = t < b && L[t][t] > 0.0 ? 1.0 / L[t][t] : 0.0;
}

// X <- X L^-T row by row (the CholeskyQR step's orthonormalization): y L^T = x, i.e.
// y_i = (x_i - sum_{k<i} L[i][k] y_k) / L[i][i] in binary64, 0 where the pivot is not
// positive.  One wave per row, lane j holding x_j: step i takes y_i from lane i and subtracts
// L[j][i] y_i from the lanes j > i, so each x_j gets its terms in increasing i.  Sixteen rows
// per block share L^T in LDS.
constexpr int kSolveRows = 16;
__global__ __launch_bounds__(64 * kSolveRows) void solve_rows_kernel(float* __restrict__ X, int rows, int b,
                                                                     const double* __restrict__ lt,
                                                                     const double* __restrict__ invd) {
    __shared__ double Lt[kW][kW];   // Lt[i][j] = L[j][i]
    __shared__ double id[kW];
    const int tid = threadIdx.x, lane = tid & 63;
    for (int e = tid; e < kW * kW; e += 64 * kSolveRows) Lt[e >> 6][e & 63] = lt[e];
    if (tid < kW) id[tid] = invd[tid];
    __syncthreads();
    const int64_t r = (int64_t)blockIdx.x * kSolveRows + (tid >> 6);
    if (r >= rows) return;   // a whole wave
    double x = X[r * kW + lane];
    double y = 0.0;
    for (int i = 0; i < b; ++i) {
        const double yi = readlane_f64(x, i) * id[i];
        if (lane == i) y = yi;
        if (lane > i) x -= Lt[i][lane] * yi;
    }
    X[r * kW + lane] = (float)y;
}

// Z^T Z = U_B diag(sigma^2) U_B^T by cyclic Jacobi (binary64, kJacobiThreads threads: the
// rotations of a round are applied by all of them), eigenvalues sorted in decreasing order:
// ub[i][j] (64 x 64, the first r columns used), sigma[j] = sqrt(ev_j).
constexpr int kJacobiThreads = 1024;
__global__ __launch_bounds__(kJacobiThreads) void jacobi_kernel(const double* __restrict__ gram, int b,
                                                                float* __restrict__ ub, float* __restrict__ sigma) {
    __shared__ double S[kW][kW + 1];   // padded: column walks stay conflict-free
    __shared__ double V[kW][kW + 1];   // padded: column walks stay conflict-free
    __shared__ int order[kW];
    __shared__ int pp[kW / 2], pq[kW / 2];
    __shared__ double pc[kW / 2], ps[kW / 2];
    const int t = threadIdx.x;
    load_gram(gram, b, S);
    if (t < kW)
        for (int i = 0; i < kW; ++i) V[i][t] = i == t ? 1.0 : 0.0;
    __syncthreads();
    // Parallel cyclic Jacobi, round-robin ordering: with nb = b rounded up to even, a sweep
    // is nb - 1 rounds; round r pairs the positions i and nb - 1 - i of the list
    // (0, 1 + (r mod (nb - 1)), ...), so every index pair meets once per sweep and the
    // pairs of a round are disjoint.  Each round takes every pair's rotation from S as the
    // round finds it, then applies all of them: columns (S and V), then rows.
    const int nb = (b + 1) & ~1, np = nb / 2;
    __shared__ double red[2][kJacobiThreads], red2[2][32];
    __shared__ int stop;
    // the round-robin schedule: round rd pairs the positions i and nb - 1 - i of the list
    // (0, 1 + (rd mod (nb - 1)), ...), p < q
    __shared__ uint8_t tp[kW][kW / 2], tq[kW][kW / 2];
    for (int e = t; e < (nb - 1) * np; e += kJacobiThreads) {
        const int rd = e / np, i0 = e - rd * np, i1 = nb - 1 - i0;
        const int p = i0 == 0 ? 0 : 1 + (i0 - 1 + rd) % (nb - 1);
        const int q = 1 + (i1 - 1 + rd) % (nb - 1);
        tp[rd][i0] = (uint8_t)min(p, q), tq[rd][i0] = (uint8_t)max(p, q);
    }
    for (int sweep = 0; sweep < 30; ++sweep) {
        // off-diagonal and diagonal squares: each thread sums a fixed set of entries; the
        // per-thread sums are added in a fixed order
        double off = 0.0, dia = 0.0;
        for (int e = t; e < b * b; e += kJacobiThreads) {
            const int i = e / b, j = e - i * b;
            (i == j ? dia : off) += S[i][j] * S[i][j];
        }
        red[0][t] = off, red[1][t] = dia;
        __syncthreads();
        if (t < 32) {   // 32 runs of consecutive threads, each summed in order, then the runs
            double o = 0.0, d = 0.0;
            for (int k = 0; k < kJacobiThreads / 32; ++k) o += red[0][t * (kJacobiThreads / 32) + k],
                                                           d += red[1][t * (kJacobiThreads / 32) + k];
            red2[0][t] = o, red2[1][t] = d;
        }
        __syncthreads();
        if (t == 0) {
            double o = 0.0, d = 0.0;
            for (int k = 0; k < 32; ++k) o += red2[0][k], d += red2[1][k];
            stop = o <= 1e-24 * d;
        }
        __syncthreads();
        if (stop) break;
        for (int rd = 0; rd < nb - 1; ++rd) {
            if (t < np) {
                const int p = tp[rd][t], q = tq[rd][t];
                double c = 1.0, sn = 0.0;
                if (q < b) {
                    const double apq = S[p][q];
                    if (fabs(apq) > 1e-300) {
                        const double th = (S[q][q] - S[p][p]) / (2.0 * apq);
                        // tan of the angle; 1 / (2 th) where th * th would overflow
                        const double tt = fabs(th) > 1e150
                                              ? 0.5 / th
                                              : (th >= 0.0 ? 1.0 : -1.0) / (fabs(th) + __builtin_sqrt(th * th + 1.0));
                        c = 1.0 / __builtin_sqrt(tt * tt + 1.0);
                        sn = tt * c;
                    }
                }
                pp[t] = p, pq[t] = q, pc[t] = c, ps[t] = sn;
            }
            __syncthreads();
            // S <- J^T S J and V <- V J in one pass.  J rotates each pair (p, q) of the round:
            // column p <- c col p - s col q, column q <- s col p + c col q, and rows alike.
            // The pairs cover every index, so S splits into 2 x 2 blocks (rows of pair a,
            // columns of pair e), each updated from its own old values: columns first, then
            // rows -- the same operations, in the same order, as rotating all columns and
            // then all rows.
            for (int it = t; it < 32 * 32 + 32 * kW; it += kJacobiThreads) {
                if (it < 32 * 32) {
                    const int a = it >> 5, e = it & 31;
                    if (a >= np || e >= np) continue;
                    const double sa = ps[a], se = ps[e];
                    if (sa == 0.0 && se == 0.0) continue;
                    const int pa = pp[a], qa = pq[a], pe = pp[e], qe = pq[e];
                    double m00 = S[pa][pe], m01 = S[pa][qe], m10 = S[qa][pe], m11 = S[qa][qe];
                    if (se != 0.0) {
                        const double ce = pc[e];
                        const double n00 = ce * m00 - se * m01, n01 = se * m00 + ce * m01;
                        const double n10 = ce * m10 - se * m11, n11 = se * m10 + ce * m11;
                        m00 = n00, m01 = n01, m10 = n10, m11 = n11;
                    }
                    if (sa != 0.0) {
                        const double ca = pc[a];
                        const double n00 = ca * m00 - sa * m10, n10 = sa * m00 + ca * m10;
                        const double n01 = ca * m01 - sa * m11, n11 = sa * m01 + ca * m11;
                        m00 = n00, m01 = n01, m10 = n10, m11 = n11;
                    }
                    S[pa][pe] = m00, S[pa][qe] = m01, S[qa][pe] = m10, S[qa][qe] = m11;
                } else {
                    const int u = it - 32 * 32, pr = u >> 6, k = u & 63;
                    if (pr >= np || k >= b) continue;
                    const double sn = ps[pr];
                    if (sn == 0.0) continue;
                    const int p = pp[pr], q = pq[pr];
                    const double c = pc[pr];
                    const double vp = V[k][p], vq = V[k][q];
                    V[k][p] = c * vp - sn * vq;
                    V[k][q] = sn * vp + c * vq;
                }
            }
            __syncthreads();
        }
    }
    if (t == 0) {   // order by decreasing eigenvalue (selection)
        for (int i = 0; i < b; ++i) order[i] = i;
        for (int i = 0; i < b; ++i) {
            int m = i;
            for (int j = i + 1; j < b; ++j)
                if (S[order[j]][order[j]] > S[order[m]][order[m]]) m = j;
            const int tmp = order[i];
            order[i] = order[m], order[m] = tmp;
        }
    }
    __syncthreads();
    if (t < kW)
        for (int i = 0; i < kW; ++i) ub[i * kW + t] = t < b && i < b ? (float)V[i][order[t]] : 0.0f;
    if (t < b) sigma[t] = (float)__builtin_sqrt(fmax(S[order[t]][order[t]], 0.0));
}

// l2[n, j] = bf16((Q U_B)[n, j] sqrt(sigma_j)); l1[j, k] = bf16((Z U_B)[k, j] smooth_inv[k]
// / sqrt(sigma_j)) (V = Z U_B / sigma, times sqrt(sigma)).  One thread per element.
__global__ __launch_bounds__(256) void factors_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ Z,
                                                      const float* __restrict__ ub,
                                                      const float* __restrict__ sigma,
                                                      const float* __restrict__ smooth_inv, int N,
                                                      int K, int r, int b, uint16_t* __restrict__ l1,
                                                      uint16_t* __restrict__ l2) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t nl2 = (int64_t)N * r, nl1 = (int64_t)r * K;
    if (t >= nl2 + nl1) return;
    if (t < nl2) {
        const int n = (int)(t / r), j = (int)(t - (int64_t)n * r);
        float s = 0.0f;
        for (int i = 0; i < b; ++i) s = fmaf(Q[(int64_t)n * kW + i], ub[i * kW + j], s);
        l2[t] = (uint16_t)f32_to_bf16(s * sqrtf(sigma[j]));
    } else {
        const int64_t u = t - nl2;
        const int j = (int)(u / K), k = (int)(u - (int64_t)j * K);
        float s = 0.0f;
        for (int i = 0; i < b; ++i) s = fmaf(Z[(int64_t)k * kW + i], ub[i * kW + j], s);
        const float sg = sigma[j];
        l1[u] = (uint16_t)f32_to_bf16(sg > 0.0f ? s * smooth_inv[k] / sqrtf(sg) : 0.0f);
    }
}

// dst [rows, 64] <- src [rows, b], columns past b zero
__global__ __launch_bounds__(256) void pad_kernel(const float* __restrict__ src, int rows, int b,
                                                  float* __restrict__ dst) {
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)rows * kW) return;
    const int64_t r = t / kW;
    const int j = (int)(t - r * kW);
    dst[t] = j < b ? src[r * b + j] : 0.0f;
}

constexpr int kSlices = 20;  // inner-dimension slices of a skinny product (enough blocks to fill the GPU)

struct Work {
    float *Q, *Z, *ub, *sigma, *slices;
    double *part, *gsum, *lt, *invd;
};

Work carve(void* ws, int N, int K) {
    const int nblk = (std::max(N, K) + kGramRows - 1) / kGramRows;
    uint8_t* p = (uint8_t*)ws;
    Work w;
    w.part = (double*)p;
    p += (int64_t)nblk * kW * kW * 8;
    w.gsum = (double*)p;
    p += (int64_t)kW * kW * 8;
    w.slices = (float*)p;
    p += (int64_t)kSlices * std::max(N, K) * kW * 4;
    w.Q = (float*)p;
    p += (int64_t)N * kW * 4;
    w.Z = (float*)p;
    p += (int64_t)K * kW * 4;
    w.lt = (double*)p;
    p += kW * kW * 8;
    w.invd = (double*)p;
    p += kW * 8;
    w.ub = (float*)p;
    p += kW * kW * 4;
    w.sigma = (float*)p;
    return w;
}

// Y = W_hat X (TRANS false, Y [N, 64]) or W_hat^T X (TRANS true, Y [K, 64])
template <bool TRANS>
void skinny(const float* W, const float* smooth_inv, int N, int K, const float* X, float* Y,
            const Work& w, hipStream_t st) {
    const int rows = TRANS ? K : N, inner = TRANS ? N : K;
    const int chunk = ((inner + kSlices - 1) / kSlices + 31) / 32 * 32;
    const int slices = (inner + chunk - 1) / chunk;
    hipLaunchKernelGGL(skinny_kernel<TRANS>, dim3((unsigned)((rows + kW - 1) / kW), (unsigned)slices), dim3(256),
                       0, st, W, smooth_inv, N, K, X, chunk, w.slices);
    const int64_t n = (int64_t)rows * kW;
    hipLaunchKernelGGL(sum_slices_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float*)w.slices, n, slices, Y);
}

void orth(float* X, int rows, int b, const Work& w, hipStream_t st) {
    const int nblk = (rows + kGramRows - 1) / kGramRows;
    for (int pass = 0; pass < 2; ++pass) {   // CholeskyQR2
        hipLaunchKernelGGL(gram_partial_kernel, dim3(nblk), dim3(256), 0, st, (const float*)X, rows, w.part);
        hipLaunchKernelGGL(gram_sum_kernel, dim3(kW * kW / 64), dim3(64 * kGramParts), 0, st, (const double*)w.part, nblk,
                           w.gsum);
        hipLaunchKernelGGL(chol_kernel, dim3(1), dim3(64), 0, st, (const double*)w.gsum, 1, b, w.lt, w.invd);
        hipLaunchKernelGGL(solve_rows_kernel, dim3((unsigned)((rows + kSolveRows - 1) / kSolveRows)),
                           dim3(64 * kSolveRows), 0, st, X, rows, b, (const double*)w.lt, (const double*)w.invd);
    }
}

}  // namespace

int64_t lowrank_workspace_bytes(int N, int K) {
    const int nblk = (std::max(N, K) + kGramRows - 1) / kGramRows;
    return (int64_t)(nblk + 1) * kW * kW * 8 + (int64_t)kSlices * std::max(N, K) * kW * 4 +
           (int64_t)(N + K) * kW * 4 + kW * kW * 8 + kW * 8 + kW * kW * 4 + kW * 4;
}

void launch_lowrank_factors(int N, int K, int r, int b, int iters, const float* w,
                            const float* smooth_inv, const float* omega, void* l1, void* l2,
                            float* sigma_out, void* workspace, hipStream_t st) {
    const Work wk = carve(workspace, N, K);
    const dim3 gK((unsigned)((K + kGramRows - 1) / kGramRows));
    hipLaunchKernelGGL(pad_kernel, dim3((unsigned)(((int64_t)K * kW + 255) / 256)), dim3(256), 0, st, omega, K,
                       b, wk.Z);
    skinny<false>(w, smooth_inv, N, K, wk.Z, wk.Q, wk, st);
    orth(wk.Q, N, b, wk, st);
    for (int it = 0; it < iters; ++it) {
        skinny<true>(w, smooth_inv, N, K, wk.Q, wk.Z, wk, st);
        orth(wk.Z, K, b, wk, st);
        skinny<false>(w, smooth_inv, N, K, wk.Z, wk.Q, wk, st);
        orth(wk.Q, N, b, wk, st);
    }
    skinny<true>(w, smooth_inv, N, K, wk.Q, wk.Z, wk, st);
    hipLaunchKernelGGL(gram_partial_kernel, gK, dim3(256), 0, st, (const float*)wk.Z, K, wk.part);
    hipLaunchKernelGGL(gram_sum_kernel, dim3(kW * kW / 64), dim3(64 * kGramParts), 0, st, (const double*)wk.part, (int)gK.x,
                       wk.gsum);
    hipLaunchKernelGGL(jacobi_kernel, dim3(1), dim3(kJacobiThreads), 0, st, (const double*)wk.gsum, b, wk.ub,
                       wk.sigma);
    const int64_t tot = (int64_t)N * r + (int64_t)r * K;
    hipLaunchKernelGGL(factors_kernel, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st,
                       (const float*)wk.Q, (const float*)wk.Z, (const float*)wk.ub, (const float*)wk.sigma,
                       smooth_inv, N, K, r, b, (uint16_t*)l1, (uint16_t*)l2);
    // a failed copy leaves its error as the thread's last HIP error, which the API call
    // reports right after this launcher returns
    if (sigma_out) (void)hipMemcpyAsync(sigma_out, wk.sigma, (size_t)r * 4, hipMemcpyDeviceToDevice, st);
}

}  // namespace svdq

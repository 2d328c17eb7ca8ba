// packed_layout.hpp -- MFMA-ready operand layouts of the fast INT4 W4A4 path (gfx950).
//
// Both GEMM operands are stored as signed FP6 E2M3 fragments of the 32x32x64 f8f6f4 MFMA:
// an int4 code q in [-8, 7] is the FP6 field sign << 5 | |q|, whose value is exactly q / 8
// (|q| < 8 is a subnormal m/8, |q| = 8 is the smallest normal 1.0).  A fragment covers 32
// rows (activations) or 32 columns (weights) and one 64-channel group; MFMA lane L holds
// row/column L % 32 and channels 32 * (L / 32) + j, j = 0..31, field j at bit 6 j of six
// dwords.  The six dwords are stored as two planes so that every lane reads with one
// 16-byte and one 8-byte access, both conflict-free in LDS:
//   bytes [0, 1024)     dwords 0-3 of lane L at 16 L
//   bytes [1024, 1536)  dwords 4-5 of lane L at 1024 + 8 L
// followed by the operand of the bf16 scale MFMA (v_mfma_f32_32x32x8_bf16), which forms the
// outer product sa[m] * 64 sw[n] from bf16 hi/lo splits (hi = bf16(s), lo = bf16(s - hi)):
//   activations: 32 words (sa_hi | sa_lo << 16), one per row               (128 bytes)
//   weights:     64 lane pairs; lanes 0-31 (w_hi | w_hi << 16, w_lo) for column L with
//                w = 64 sw, lanes 32-63 zero                               (512 bytes)
// so that sum_k A[m,k] B[k,n] = sa_hi w_hi + sa_lo w_hi + sa_hi w_lo.
//
// Activation buffer:  [ceil(M / 256)][G][8 row blocks][1664 bytes]
// Weight buffer:      [ceil(N / 192)][G][6 column blocks][2048 bytes]
// One (256-row block, group) is 13 KiB and one (192-column block, group) 12 KiB, each
// contiguous, which is what one GEMM pipeline stage copies.
#pragma once

#include <stdint.h>

namespace svdq {
namespace packed {

constexpr int kBM = 256, kBN = 192;      // GEMM output tile per workgroup
constexpr int kRB = kBM / 32;            // row blocks per tile
constexpr int kCB = kBN / 32;            // column blocks per tile
constexpr int kFrag = 1536;              // FP6 fragment bytes
constexpr int kABlock = kFrag + 128;     // activation block: fragment + 32 scale words
constexpr int kBBlock = kFrag + 512;     // weight block: fragment + 64 scale pairs
constexpr int kAStage = kRB * kABlock;   // 13312
constexpr int kBStage = kCB * kBBlock;   // 12288

__host__ __device__ inline int64_t act_bytes(int64_t M, int K) {
    return (M + kBM - 1) / kBM * (int64_t)(K / 64) * kAStage;
}
__host__ __device__ inline int64_t wgt_bytes(int N, int K) {
    return (int64_t)((N + kBN - 1) / kBN) * (K / 64) * kBStage;
}

// Byte offset of the activation block holding row m of group g (G groups).
__host__ __device__ inline int64_t act_block(int64_t m, int g, int G) {
    return ((m / kBM) * G + g) * (int64_t)kAStage + ((m % kBM) / 32) * kABlock;
}
// Byte offset of the weight block holding column n of group g.
__host__ __device__ inline int64_t wgt_block(int n, int g, int G) {
    return ((int64_t)(n / kBN) * G + g) * kBStage + ((n % kBN) / 32) * kBBlock;
}
// Byte offset, inside a block, of fragment dword d (0..5) of lane L.
__host__ __device__ inline int frag_dword(int L, int d) {
    return d < 4 ? 16 * L + 4 * d : 1024 + 8 * L + 4 * (d - 4);
}

}  // namespace packed
}  // namespace svdq

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
// followed by the operands of the bf16 scale MFMA (v_mfma_f32_32x32x8_bf16), which forms
// the outer product sa[m] * w[n], w = 64 sw, from three-term bf16 splits
// (h = bf16(s), m = bf16(s - h), l = bf16(s - h - m); h + m + l = s to ~2^-27):
//   activations: per row (h | h << 16, m | l << 16) = the bf16 values (h, h, m, l), read
//                as they are by both halves of the MFMA's lanes               (256 bytes)
//   weights:     per MFMA lane, lanes 0-31 (column L) (h | m << 16, h | h << 16) = (h, m, h, h),
//                lanes 32-63 (column L - 32) (l, m | m << 16) = (l, 0, m, m)    (512 bytes)
// so that the eight products (k = 0..3 from lanes 0-31, k = 4..7 from lanes 32-63) are
// ha hw, ha mw, ma hw, la hw, ha lw, 0, ma mw, la mw and sum to
// (ha + ma + la)(hw + mw + lw) - ma lw - la lw: the fp32 product to a few ulp (the two
// dropped terms are below 2^-26 of it).
//
// Activation buffer:  [ceil(M / 256)][G][8 row blocks][1792 bytes]
// Weight buffer:      [ceil(N / 192)][G][6 column blocks][2048 bytes]
// One (256-row block, group) is 14 KiB and one (192-column block, group) 12 KiB, each
// contiguous, which is what one GEMM pipeline stage copies.
#pragma once

#include <stdint.h>

#include "common.hpp"

namespace svdq {
namespace packed {

constexpr int kBM = 256, kBN = 192;      // GEMM output tile per workgroup
constexpr int kRB = kBM / 32;            // row blocks per tile
constexpr int kCB = kBN / 32;            // column blocks per tile
constexpr int kFrag = 1536;              // FP6 fragment bytes
constexpr int kABlock = kFrag + 256;     // activation block: fragment + 32 scale pairs
constexpr int kBBlock = kFrag + 512;     // weight block: fragment + 64 scale pairs
constexpr int kAStage = kRB * kABlock;   // 14336
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

// Three-term bf16 split of s: h = bf16(s), m = bf16(s - h), l = bf16(s - h - m); both
// subtractions are exact in fp32.
__device__ __forceinline__ void split3(float s, uint32_t& h, uint32_t& m, uint32_t& l) {
    h = f32_to_bf16(s);
    const float r1 = s - __uint_as_float(h << 16);
    m = f32_to_bf16(r1);
    l = f32_to_bf16(r1 - __uint_as_float(m << 16));
}

// The activation scale pair of one row: (h | h << 16, m | l << 16).
__device__ __forceinline__ uint2 act_scale_pair(float s) {
    uint32_t h, m, l;
    split3(s, h, m, l);
    return make_uint2(h | (h << 16), m | (l << 16));
}

// The weight scale operand of MFMA lane L for w = 64 sw of its column.
__device__ __forceinline__ uint2 wgt_scale_operand(float w, int L) {
    uint32_t h, m, l;
    split3(w, h, m, l);
    return L < 32 ? make_uint2(h | (m << 16), h | (h << 16)) : make_uint2(l, m | (m << 16));
}

}  // namespace packed
}  // namespace svdq

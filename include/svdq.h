/*
 * svdq.h -- C ABI of the MI355X (gfx950) SVDQuant W4A4 / AWQ W4A16 linear library.
 *
 * The operation (pages, in their own words restated):
 *   [margrop] "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers" (blog.margrop.com),
 *             技术细节 1, "SVDQuant 的核心思路": activation outliers are migrated into the
 *             weights; the hardest part of each weight is kept as a 16-bit low-rank branch;
 *             the residual runs with 4-bit weights and activations; the low-rank
 *             down-projection is fused into the quantization kernel and the up-projection
 *             into the 4-bit compute kernel.
 *   [margrop] 技术细节 3: kernel families svdq_w4a4 (precision int4 or nvfp4) and
 *             awq_w4a16 (int4); loading on an unsupported GPU fails with a clear error and
 *             never returns wrong results.
 *   [ainews]  "Diffusers Natively Integrates Nunchaku Lite, Using W4A4 ...", paragraphs 2-3:
 *             config.json records method, precision, group size, low-rank rank and target
 *             modules; attention/MLP projections use SVDQ W4A4, modulation layers AWQ W4A16.
 *
 * A linear layer y = x W^T + b runs as two calls:
 *   svdq_quantize_act : x (bf16) -> 4-bit codes + scales of x * diag(smooth_inv), and
 *                       lora_act = x . L1^T (bf16), in one pass over x;
 *   svdq_gemm_w4a4    : y = dequant(codes_x) . dequant(codes_w)^T + lora_act . L2^T + b
 *                       (optionally GELU-tanh), fp32 or bf16 output.
 * and the modulation layers as one call, awq_gemm_w4a16.
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller allocates and owns every buffer (device memory unless stated).
 *     The library allocates nothing, keeps no pointer after a call returns, and enqueues
 *     its work asynchronously on `stream` (0 = the null stream); buffers must stay alive
 *     until that work completes.
 *   - Layouts are row-major and dense.  "bf16" is the 16-bit brain float, passed as raw
 *     16-bit words.
 *   - Errors: every function validates its arguments before launching anything and returns
 *     a status; on a non-OK status nothing was enqueued.  A thread-local message with the
 *     detail is available from svdq_last_error().  Faults inside a kernel surface, as for
 *     any HIP work, at the caller's next synchronisation.
 *   - Device: the current HIP device must be an MI355X-class gfx950 GPU; any other device
 *     yields SVDQ_ERR_UNSUPPORTED_DEVICE (checked once per device and cached).
 *   - M = 0 is valid and enqueues nothing.
 */
#ifndef SVDQ_H
#define SVDQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* svdq_stream_t;   /* same type as hipStream_t */

typedef enum {
    SVDQ_OK = 0,
    SVDQ_ERR_INVALID_ARG = 1,        /* bad shape, null or misaligned pointer, bad enum */
    SVDQ_ERR_UNSUPPORTED_DEVICE = 2, /* current device is not gfx950 */
    SVDQ_ERR_UNSUPPORTED_CONFIG = 3, /* well-formed but not implemented (e.g. rank > 128) */
    SVDQ_ERR_LAUNCH = 4              /* the HIP runtime refused a launch */
} svdq_status;

typedef enum { SVDQ_PREC_INT4 = 0, SVDQ_PREC_NVFP4 = 1 } svdq_precision;
typedef enum { SVDQ_DT_F32 = 0, SVDQ_DT_BF16 = 1 } svdq_dtype;
typedef enum { SVDQ_ACT_NONE = 0, SVDQ_ACT_GELU_TANH = 1 } svdq_act;

/* The quantization fields a checkpoint's config.json records for one layer
 * ([ainews] paragraph 2: method, precision, group size, low-rank rank). */
typedef struct {
    int32_t in_features;   /* K: a positive multiple of 64 */
    int32_t out_features;  /* N: >= 1 */
    int32_t rank;          /* r: 0, or a multiple of 16 up to 128 */
    int32_t group_size;    /* 64 for INT4, 16 for NVFP4 */
    int32_t precision;     /* svdq_precision */
} svdq_layer_cfg;

/*
 * svdq_quantize_act -- the activation kernel of an SVDQ W4A4 layer.
 * ([margrop] 技术细节 1 steps 1, 3 and 4.)
 *
 *   x          [M, K] bf16, device.                      Read only.
 *   smooth_inv [K] fp32, device: 1/lambda per input channel (outliers migrated to W).
 *   l1         [r, K] bf16, device, the low-rank down factor with 1/lambda absorbed;
 *              may be NULL when r == 0.
 *   act_global_scale  NVFP4 only: the activation's per-tensor fp32 scale S_a (> 0, finite);
 *              ignored for INT4.
 *   act_codes  [M, K/2] bytes, device, written: two 4-bit codes per byte, the even
 *              channel in the low nibble.  INT4: two's-complement codes
 *              q = clamp(rne(x_hat / s), -8, 7) with x_hat = fp32(x) * smooth_inv (one
 *              fp32 multiply), s = absmax_group(|x_hat|) / 7 (fp32 division), groups of 64
 *              channels, q = 0 where s = 0 (codes are always in [-7, 7]).
 *              NVFP4: E2M1 codes (sign in bit 3) of x_hat / (sb * S_a) rounded to nearest,
 *              ties to even, saturating at 6, per block of 16 channels.
 *   act_scales INT4: [M, K/64] fp32 s.  NVFP4: [M, K/16] E4M3 bytes
 *              sb = E4M3(min(absmax / (6 * S_a), 448)) (nearest, ties to even); codes are 0
 *              where sb = 0.  Device, written.
 *   lora_act   [M, r] bf16, device, written: bf16(sum_k x[m,k] * l1[j,k]) accumulated in
 *              fp32 (may differ from a correctly rounded fp64 sum by one bf16 ulp).
 *              May be NULL when r == 0.
 * Pointers must be 16-byte aligned.  Quantized codes and scales are bit-exact functions
 * of the inputs (no dependence on launch shape or run).
 */
svdq_status svdq_quantize_act(const svdq_layer_cfg* cfg, int64_t M, const void* x,
                              const float* smooth_inv, const void* l1,
                              float act_global_scale, void* act_codes, void* act_scales,
                              void* lora_act, svdq_stream_t stream);

/*
 * svdq_gemm_w4a4 -- the 4-bit x 4-bit GEMM of an SVDQ W4A4 layer with the low-rank
 * up-projection and bias in its epilogue ([margrop] 技术细节 1 step 4).
 *
 *   act_codes, act_scales, act_global_scale : as written by svdq_quantize_act.
 *   wgt_codes  [N, K/2] bytes: the residual weight codes, same format as act_codes
 *              (INT4 codes must lie in [-8, 7]; NVFP4 codes any E2M1 value).
 *   wgt_scales INT4: [N, K/64] fp32.  NVFP4: [N, K/16] E4M3 bytes.
 *   wgt_global_scale  NVFP4 only: S_w (> 0, finite); ignored for INT4.
 *   lora_act   [M, r] bf16 (from svdq_quantize_act); l2 [N, r] bf16, the up factor.
 *              Both may be NULL when r == 0.
 *   bias       [N] bf16 or NULL.
 *   act        svdq_act: SVDQ_ACT_GELU_TANH applies 0.5 y (1 + tanh(sqrt(2/pi)(y + 0.044715 y^3)))
 *              after the bias (the fused GELU of a DiT MLP's first linear).
 *   out_dtype  svdq_dtype of `out`.
 *   out        [M, N] device, written:
 *              INT4:  y = sum_g sa[m,g] sw[n,g] sum_{k in g} qa[m,k] qw[n,k]
 *              NVFP4: y = S_a S_w sum_k e_a[m,k] sb_a[m,k/16] e_w[n,k] sb_w[n,k/16]
 *              plus sum_j lora_act[m,j] l2[n,j] + bias[n], accumulated in fp32.
 * For INT4 this call is the reference path on the plain nibble format: it contracts the
 * nibbles on the int8 MFMA with 128x128 tiles (about 151 us at M = 4096, K = N = 3072 on
 * an MI355X).  The primary INT4 path is the packed one below (svdq_prepack_weight once per
 * layer, svdq_quantize_act_packed, svdq_gemm_w4a4_packed: about 42 us for that GEMM), with
 * the same result up to fp32 rounding order.
 */
svdq_status svdq_gemm_w4a4(const svdq_layer_cfg* cfg, int64_t M, const void* act_codes,
                           const void* act_scales, float act_global_scale,
                           const void* wgt_codes, const void* wgt_scales,
                           float wgt_global_scale, const void* lora_act, const void* l2,
                           const void* bias, int32_t act, int32_t out_dtype, void* out,
                           svdq_stream_t stream);

/*
 * awq_gemm_w4a16 -- AWQ W4A16 GEMV / skinny GEMM for modulation layers ([ainews]
 * paragraph 3; [margrop] 技术细节 3, awq_w4a16 int4).
 *
 *   x        [M, K] bf16 (the per-channel AWQ scale already folded into x).
 *   qweight  [N, K/2] bytes: unsigned 4-bit q, even channel in the low nibble.
 *   scales   [N, K/group_size] bf16;  zeros [N, K/group_size] bf16 (integer values).
 *   bias     [N] bf16 or NULL.
 *   out      [M, N] fp32 or bf16: y = sum_k x[m,k] (q[n,k] - z[n,g]) s[n,g] + bias[n],
 *            accumulated in fp32.
 * group_size must be 64; K a multiple of 64; any M >= 0 (one pass over the weights
 * serves up to 4 rows; larger M re-reads them).
 */
svdq_status awq_gemm_w4a16(int64_t M, int32_t K, int32_t N, int32_t group_size, const void* x,
                           const void* qweight, const void* scales, const void* zeros,
                           const void* bias, int32_t out_dtype, void* out,
                           svdq_stream_t stream);

/*
 * Packed INT4 operands -- the fast GEMM path ([margrop] 技术细节 1 steps 3-4: the quantize
 * kernel hands the GEMM its 4-bit operands in the layout the matrix unit consumes).
 * Both operands are stored as exact FP6 (E2M3) values q/8 of the int4 codes in the lane
 * order of the gfx950 32x32x64 FP6 MFMA, 32 rows (or columns) x 64 channels per fragment,
 * each followed by the group scales as three-term bf16 splits (h = bf16(s), m = bf16(s - h),
 * l = bf16(s - h - m), h + m + l = s to ~2^-27) arranged as operands of a bf16 MFMA that
 * forms the scale products.  Activations take 6 bits per code plus 8 bytes per (row, group)
 * and are padded to a multiple of 256 rows; weights take 6 bits per code plus 16 bytes per
 * (column, group) and are padded to a multiple of 192 columns.  The buffers are opaque;
 * sizes come from the *_bytes queries.  All buffers are device memory, 16-byte aligned,
 * owned by the caller.
 *
 * svdq_act_packed_bytes / svdq_prepacked_weight_bytes: buffer sizes for `cfg` (INT4 only)
 *   and M rows.
 * svdq_prepacked_l1_bytes: buffer size of the prepacked low-rank factor for `cfg`
 *   (ceil(K / 128) * 128 * rank * 2 bytes; 0 at rank 0).
 * svdq_prepack_l1: the low-rank down-projection factor l1 bf16 [rank, K] row-major ->
 *   l1_packed, reordered so the activation kernel reads each of its MFMA operands as one
 *   contiguous 1 KiB (a layout detail of this library; the values are l1's, channels past
 *   K are zero).  Once per layer, like the weight prepack.  A no-op at rank 0.
 * svdq_quantize_act_packed: as svdq_quantize_act (INT4), writing the codes into act_packed
 *   instead of nibbles and taking the low-rank factor as l1_packed (svdq_prepack_l1
 *   output; may be NULL at rank 0); the codes, the fp32 scales (act_scales, may be NULL)
 *   and lora_act are bit-identical to svdq_quantize_act's on the unpacked l1.  Padding rows
 *   of act_packed are zero.
 * svdq_pack_act: act_codes [M, K/2] nibbles + act_scales [M, K/64] fp32 (svdq_quantize_act
 *   output) -> act_packed.
 * svdq_prepack_weight: wgt_codes [N, K/2] nibbles (full range [-8, 7]) + wgt_scales
 *   [N, K/64] fp32 -> prepacked, once per layer.
 * svdq_gemm_w4a4_packed: as svdq_gemm_w4a4 (INT4) on packed operands.  The result equals
 *   svdq_gemm_w4a4's up to fp32 rounding order and the three-term split of each scale
 *   product (relative error of one group's scale product a few fp32 ulp).  The output is
 *   computed in 256x192 tiles, one per compute unit at a time, each summed over the groups
 *   in a fixed order: the result is bit-reproducible from run to run.
 * svdq_gemm_w4a4_packed_workspace_bytes: the workspace svdq_gemm_w4a4_packed_ws uses for
 *   this layer, M rows, `act` and `out_dtype` (0 when it would not split; at most 64 MiB).
 * svdq_gemm_w4a4_packed_ws: svdq_gemm_w4a4_packed with a caller-owned device workspace
 *   (16-byte aligned, workspace_bytes long, contents overwritten; may be NULL with
 *   workspace_bytes 0).  With fp32 output and no activation, when the last round of tiles
 *   would fill at most a quarter of the compute units, those tiles are split over K into
 *   up to 8 parts (as many as the workspace holds, at least 2, else no split): each part
 *   stores its fp32 partial tile in the workspace and a second kernel adds the parts in the
 *   fixed order of their K ranges.  Bit-reproducible from run to run for a given workspace
 *   size; it differs from svdq_gemm_w4a4_packed's output only in the fp32 order of the sum.
 * All enqueue on `stream`.
 */
svdq_status svdq_act_packed_bytes(const svdq_layer_cfg* cfg, int64_t M, int64_t* bytes);
svdq_status svdq_prepacked_weight_bytes(const svdq_layer_cfg* cfg, int64_t* bytes);
svdq_status svdq_prepacked_l1_bytes(const svdq_layer_cfg* cfg, int64_t* bytes);
svdq_status svdq_prepack_l1(const svdq_layer_cfg* cfg, const void* l1, void* l1_packed,
                            svdq_stream_t stream);
svdq_status svdq_quantize_act_packed(const svdq_layer_cfg* cfg, int64_t M, const void* x,
                                     const float* smooth_inv, const void* l1_packed,
                                     void* act_packed, float* act_scales, void* lora_act,
                                     svdq_stream_t stream);
svdq_status svdq_pack_act(const svdq_layer_cfg* cfg, int64_t M, const void* act_codes,
                          const float* act_scales, void* act_packed, svdq_stream_t stream);
svdq_status svdq_prepack_weight(const svdq_layer_cfg* cfg, const void* wgt_codes,
                                const void* wgt_scales, void* prepacked, svdq_stream_t stream);
svdq_status svdq_gemm_w4a4_packed(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                  const void* prepacked, const void* lora_act, const void* l2,
                                  const void* bias, int32_t act, int32_t out_dtype, void* out,
                                  svdq_stream_t stream);
svdq_status svdq_gemm_w4a4_packed_workspace_bytes(const svdq_layer_cfg* cfg, int64_t M, int32_t act,
                                                  int32_t out_dtype, int64_t* bytes);
svdq_status svdq_gemm_w4a4_packed_ws(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                     const void* prepacked, const void* lora_act, const void* l2,
                                     const void* bias, int32_t act, int32_t out_dtype, void* out,
                                     void* workspace, int64_t workspace_bytes, svdq_stream_t stream);

/* svdq_gemm_w4a4_packed_noalloc -- for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * computation as svdq_gemm_w4a4_packed_ws given svdq_gemm_w4a4_packed_workspace_bytes
 * bytes of workspace (same split, same fixed-order sum, same bits), with the workspace taken
 * from a 64 MiB device array inside the library instead of from the caller.  Each GPU the
 * library runs on holds that array until the process ends; the call allocates nothing.
 * All calls on one GPU share it and each call leaves its partial tiles in it: calls that
 * may run at the same time on one GPU (different streams without ordering) race and must
 * not be issued.  A split that would need more than the array holds is rejected with
 * SVDQ_ERR_UNSUPPORTED_CONFIG (the split count is capped so that this does not happen on
 * GPUs of up to 256 compute units).  Other arguments, results and errors as
 * svdq_gemm_w4a4_packed. */
svdq_status svdq_gemm_w4a4_packed_noalloc(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                          const void* prepacked, const void* lora_act, const void* l2,
                                          const void* bias, int32_t act, int32_t out_dtype, void* out,
                                          svdq_stream_t stream);

/* Two chained linears on the packed path with the second one's activation kernel fused into
 * the first one's GEMM (the DiT MLP: fc1 with GELU, then fc2).  The pages credit the original
 * engine's extra speed to such per-architecture fusions of the GELU/MLP kernels (page
 * "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 2; page "Diffusers
 * integra Nunchaku ...", the section on why the original engine is still faster).  Same
 * results as
 *
 *   svdq_gemm_w4a4_packed(cfg, M, act_packed, prepacked, lora_act, l2, bias, act,
 *                         SVDQ_DT_BF16, h)
 *   svdq_quantize_act_packed(next_cfg, M, h, next_smooth_inv, prepack(next_l1),
 *                            next_act_packed, next_act_scales, next_lora_act)
 *
 * without the bf16 activations h [M, cfg->out_features] ever reaching memory: each output
 * tile is quantized in the GEMM's epilogue from the bf16 values it would store.  Codes,
 * scale words and next_act_scales are bit-identical to the unfused pair; next_lora_act
 * (bf16 [M, next rank]) is the same sum in another fp32 order: each 192-column tile stores
 * its fp32 partial sums in lora_workspace and a second kernel adds the tiles' partials in
 * a fixed order (eight consecutive runs of tiles, each summed in column order, then the
 * runs in order) and rounds once, so it is bit-reproducible; like the unfused pair's, each
 * element lies within the fp32 error bound of the exact sum (the two differ only where
 * that bound straddles a bf16 rounding boundary).
 * next_cfg->in_features must equal cfg->out_features (both INT4).  next_l1 is the next
 * layer's row-major bf16 [rank, K] factor (not prepacked); lora_workspace is caller-owned
 * device scratch of svdq_quantize_next_workspace_bytes(cfg, next_cfg, M) bytes
 * (ceil(N / 192) * ceil(M / 256) * 256 * next rank * 4; 16-byte aligned, overwritten);
 * next_lora_act must be 8-byte aligned.  next_act_scales may be NULL; next_l1,
 * next_lora_act and lora_workspace may be NULL at next rank 0.  Enqueued on `stream`. */
svdq_status svdq_quantize_next_workspace_bytes(const svdq_layer_cfg* cfg,
                                               const svdq_layer_cfg* next_cfg, int64_t M,
                                               int64_t* bytes);
svdq_status svdq_gemm_w4a4_packed_quantize_next(
    const svdq_layer_cfg* cfg, int64_t M, const void* act_packed, const void* prepacked,
    const void* lora_act, const void* l2, const void* bias, int32_t act,
    const svdq_layer_cfg* next_cfg, const float* next_smooth_inv, const void* next_l1,
    void* next_act_packed, float* next_act_scales, void* next_lora_act, float* lora_workspace,
    svdq_stream_t stream);

/* Offline weight quantization: the calibrate-and-quantize step that turns a layer's weight
 * into the tensors the kernels above consume (page "Hugging Face 把 Nunchaku 4-bit Diffusion
 * 接到 Diffusers", 技术细节 1 "SVDQuant 的核心思路" steps 1-3 and its quantize-your-own-model
 * walk-through; page "Diffusers integra Nunchaku ...", the diffuse-compressor section).  The
 * pages give no formulas; the readings are:
 *
 * svdq_calib_absmax: absmax[k] = max(absmax[k], max_m |x[m, k]|) over bf16 calibration
 *   activations x [M, K] (K a multiple of 64); call once per batch on an absmax first
 *   filled with zeros.  Exact.
 * svdq_smoothing_factors: per input channel k of the fp32 weight w [N, K] (N = out_features),
 *   cw[k] = max_n |w[n, k]| (written to w_absmax, fp32 [K], caller-owned) and the smoothing
 *   factor lambda = sqrt(x_absmax[k] / cw[k]) in binary64, 1 where it is not a positive
 *   finite number or either maximum is 0; writes smooth_inv[k] = fp32(1 / lambda), the
 *   activation kernel's input.  Exact given the maxima (correctly rounded binary64 steps).
 * svdq_quantize_residual: with lam = 1 / smooth_inv (binary64), the 4-bit residual
 *   R = fp32(w lam - (l2 l1) lam) of the smoothed weight once the low-rank branch (l1 bf16
 *   [rank, K] with smooth_inv absorbed, l2 bf16 [N, rank], the same factors the GEMM and
 *   the activation kernel take; may be NULL at rank 0) is taken out, quantized like the
 *   activations.  INT4: wgt_codes [N, K/2] nibbles and wgt_scales [N, K/64] fp32,
 *   svdq_prepack_weight's inputs; wgt_global_scale is unused (may be NULL).  NVFP4: the
 *   per-tensor scale S_w = fp32(max |R| / 2688) is written to wgt_global_scale (one fp32
 *   in device memory, the GEMM's weight_global_scale), then wgt_codes [N, K/2] E2M1 and
 *   wgt_scales [N, K/16] E4M3 bytes under it.  The low-rank product sums bf16 products in
 *   binary64.  Each product is a 16-bit integer times 2^e_j, so the sum is exact while an
 *   element's exponents satisfy max e_j - min e_j <= 37 - ceil(log2 r) (32 at rank 32);
 *   the codes and scales are then those of the definition bit for bit.
 * svdq_lowrank_factors: the branch's factors between the two, from the leading r singular
 *   triplets of the smoothed weight W diag(lambda) (lambda = 1 / smooth_inv), split as
 *   sqrt(sigma) on each side: l2 bf16 [N, r] = U sqrt(sigma), l1 bf16 [r, K] =
 *   sqrt(sigma) V^T diag(smooth_inv); sigma (fp32 [r], may be NULL) the singular values in
 *   decreasing order.  Computed by randomized subspace iteration (Halko, Martinsson and
 *   Tropp 2011): omega is the caller's fp32 [K, block] standard-normal draws, r <= block
 *   <= 64 (oversampling block - r), `iters` power iterations (0 to 32); the result
 *   approximates the exact triplets (exact for a weight of rank <= block), closer with more
 *   oversampling and iterations.  rank 16 to 64.  workspace: device memory of
 *   svdq_lowrank_workspace_bytes(cfg) bytes, 16-byte aligned, overwritten.
 * All buffers are device memory owned by the caller; all enqueue on `stream`. */
svdq_status svdq_calib_absmax(int64_t M, int32_t K, const void* x, float* absmax,
                              svdq_stream_t stream);
svdq_status svdq_smoothing_factors(const svdq_layer_cfg* cfg, const float* w, const float* x_absmax,
                                   float* w_absmax, float* smooth_inv, svdq_stream_t stream);
svdq_status svdq_quantize_residual(const svdq_layer_cfg* cfg, const float* w, const float* smooth_inv,
                                   const void* l1, const void* l2, void* wgt_codes, void* wgt_scales,
                                   float* wgt_global_scale, svdq_stream_t stream);
svdq_status svdq_lowrank_workspace_bytes(const svdq_layer_cfg* cfg, int64_t* bytes);
svdq_status svdq_lowrank_factors(const svdq_layer_cfg* cfg, const float* w, const float* smooth_inv,
                                 const float* omega, int32_t block, int32_t iters, void* l1, void* l2,
                                 float* sigma, void* workspace, svdq_stream_t stream);

/* LoRA adapters through the low-rank branch (page "Diffusers integra Nunchaku ...",
 * "Nunchaku Lite: integración y modelo de ejecución": LoRA keeps working because the module
 * structure is kept; page "Diffusers Natively Integrates Nunchaku Lite ...", the paragraph
 * on loading through from_pretrained()).  An adapter y += alpha (x A^T) B^T is a term of the
 * branch's own form, so it is merged into the branch's factors once, after which
 * svdq_quantize_act / svdq_prepack_l1 and the GEMMs run unchanged at the merged rank:
 *
 *   l1_out [r', K] = [l1; lora_down; 0]          (bf16, row-major)
 *   l2_out [N, r'] = [l2 | bf16(alpha lora_up) | 0]
 *
 * with r = cfg->rank, lora_down = A bf16 [r_lora, K], lora_up = B bf16 [N, r_lora], and
 * r' = svdq_merged_rank(r, r_lora) = r + r_lora rounded up to a multiple of 16 (the padding
 * rows and columns are zero and add exact zeros).  alpha lora_up is one fp32 product per
 * element rounded to nearest-even bf16.  r' must not exceed 128 (else
 * SVDQ_ERR_UNSUPPORTED_CONFIG); r_lora >= 1 and alpha finite (else SVDQ_ERR_INVALID_ARG).
 * l1 and l2 may be NULL when r = 0.  Device buffers, caller-owned, 2-byte aligned;
 * enqueued on `stream`.  svdq_merged_rank returns -1 for a negative argument. */
int32_t svdq_merged_rank(int32_t rank, int32_t r_lora);
svdq_status svdq_merge_lora(const svdq_layer_cfg* cfg, int32_t r_lora, const void* l1,
                            const void* l2, const void* lora_down, const void* lora_up,
                            float alpha, void* l1_out, void* l2_out, svdq_stream_t stream);

/* SVDQ_OK when HIP device `device` is a gfx950 GPU, else SVDQ_ERR_UNSUPPORTED_DEVICE
 * (or SVDQ_ERR_INVALID_ARG for a bad ordinal).  Results are cached per device. */
svdq_status svdq_check_device(int device);

/* Host-only check of an architecture name as HIP reports it (e.g. "gfx950:sramecc+:xnack-"):
 * SVDQ_OK for gfx950, SVDQ_ERR_UNSUPPORTED_DEVICE otherwise, SVDQ_ERR_INVALID_ARG for NULL. */
svdq_status svdq_check_arch(const char* arch_name);

/* Static description of a status code. */
const char* svdq_status_string(svdq_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* svdq_last_error(void);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t svdq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SVDQ_H */

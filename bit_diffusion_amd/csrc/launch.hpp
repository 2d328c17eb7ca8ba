// launch.hpp -- host-side launchers of the gfx950 kernels (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

struct QuantArgs {
    int64_t M;
    int K, r;
    int mode;       // 0 INT4 nibbles, 1 INT4 packed (packed_layout.hpp), 2 NVFP4 nibbles
    const void* x;
    const float* smooth_inv;
    const void* l1;   // [r, K] row-major; prepacked (launch_prepack_l1) in mode 1
    float S;
    void* codes;    // nibbles, or the packed activation buffer in mode 1
    void* scales;   // may be NULL in mode 1
    void* lora;
};

struct GemmArgs {
    int64_t M;
    int N, K, r;
    bool nvfp4;
    const void* acodes;
    const void* ascales;
    float Sa;
    const void* wcodes;
    const void* wscales;
    float Sw;
    const void* lora;
    const void* l2;
    const void* bias;
    int act;        // 0 none, 1 gelu-tanh
    int out_bf16;   // 0 fp32, 1 bf16
    void* out;
};

struct AwqArgs {
    int64_t M;
    int K, N;
    const void* x;
    const void* qweight;
    const void* scales;
    const void* zeros;
    const void* bias;
    int out_bf16;
    void* out;
};

struct PackedGemmArgs {
    int64_t M;
    int N, K, r;
    const void* act;   // packed activations
    const void* wgt;   // packed weights
    const void* lora;
    const void* l2;
    const void* bias;
    int act_fn;
    int out_bf16;
    void* out;
    int vec_store;     // set by the launcher
    int nfull, nsplit, gsplit;   // K split of the last round's tiles (set by the launcher)
    // the next layer's activation quantization in the epilogue (quantize_next); the tile's
    // bf16 outputs are not stored
    int quantize_next;
    int next_r;              // next layer's rank
    const float* next_si;    // [N] smoothing factors of the next layer
    const void* next_l1;     // bf16 [next_r, N] row-major, or NULL
    void* next_packed;       // the next layer's packed activation buffer (its K = N)
    float* next_scales;      // fp32 [M, N / 64] or NULL
    float* lora_work;        // fp32 [ceil(N / 192)][ceil(M / 256) * 256][next_r]: per-tile
                             // partial sums of the next layer's low-rank down-projection
    // K split (fp32 output, no activation): workspace for the splits' partial tiles, or NULL
    // (then no split)
    float* split_ws;
    int64_t split_ws_bytes;
};

// Largest workspace the K split of svdq_gemm_w4a4_packed uses (its split count is capped so
// that the partial tiles fit).
constexpr int64_t kSplitWorkspaceMax = (int64_t)64 << 20;

void launch_quantize_act(const QuantArgs& a, hipStream_t st);
void launch_gemm_int4(const GemmArgs& a, hipStream_t st);
void launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st);
void launch_awq_gemv(const AwqArgs& a, hipStream_t st);

void launch_prepack_wgt(int N, int K, const void* wcodes, const void* wscales, void* out,
                        hipStream_t st);
void launch_merge_lora(int K, int N, int r, int rl, int ro, const void* l1, const void* l2,
                       const void* down, const void* up, float alpha, void* l1o, void* l2o,
                       hipStream_t st);
int64_t prepacked_l1_bytes(int r, int K);
void launch_prepack_l1(int r, int K, const void* l1, void* out, hipStream_t st);
void launch_pack_act(int64_t M, int K, const void* acodes, const void* ascales, void* out,
                     hipStream_t st);
bool gemm_w4a4_fp6_init();
void launch_gemm_w4a4_fp6(const PackedGemmArgs& a, hipStream_t st);
int64_t split_workspace_bytes(int64_t M, int N, int K, int act_fn, int out_bf16);
int cu_count();   // compute units of the current device (cached per device)
// device address and size of the K-split scratch array of the current device (noalloc.hip)
hipError_t noalloc_scratch(void** ptr, int64_t* bytes);

// measurement kernels (peaks.hip)
int64_t launch_mfma_peak(int kind, int iters, float* out, hipStream_t st);
void launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);
void launch_read(const void* src, int64_t bytes, void* out, hipStream_t st);
int64_t quantize_next_workspace_bytes(int64_t M, int N, int next_r);

// offline weight quantization (weights.hip)
void launch_calib_absmax(int64_t M, int K, const void* x, float* absmax, hipStream_t st);
void launch_smoothing_factors(int N, int K, const float* w, const float* x_absmax, float* w_absmax,
                              float* smooth_inv, hipStream_t st);
void launch_quantize_residual(int N, int K, int r, bool nvfp4, const float* w,
                              const float* smooth_inv, const void* l1, const void* l2, void* codes,
                              void* scales, float* global_scale, hipStream_t st);

// top-r factorization of the smoothed weight (lowrank.hip)
int64_t lowrank_workspace_bytes(int N, int K);
void launch_lowrank_factors(int N, int K, int r, int b, int iters, const float* w,
                            const float* smooth_inv, const float* omega, void* l1, void* l2,
                            float* sigma_out, void* workspace, hipStream_t st);

}  // namespace svdq

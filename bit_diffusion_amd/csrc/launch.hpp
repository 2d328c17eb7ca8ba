// launch.hpp -- host-side launchers of the gfx950 kernels (arguments already validated).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace svdq {

struct QuantArgs {
    int64_t M;
    int K, r;
    bool nvfp4;
    const void* x;
    const float* smooth_inv;
    const void* l1;
    float S;
    void* codes;
    void* scales;
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

struct PrepackedGemmArgs {
    int64_t M;
    int N, K, r;
    int ntiles_padded;
    const void* acodes;
    const void* ascales;
    const void* prepacked;
    const void* lora;
    const void* l2;
    const void* bias;
    int act;
    int out_bf16;
    void* out;
};

size_t quantize_act_lds_bytes(int K, int r);
void launch_quantize_act(const QuantArgs& a, hipStream_t st);
void launch_gemm_int4(const GemmArgs& a, hipStream_t st);
void launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st);
void launch_awq_gemv(const AwqArgs& a, hipStream_t st);

int64_t prepacked_int4_bytes(int N, int K);
int prepacked_ntiles_padded(int N);
void launch_prepack_int4(int N, int K, const void* wcodes, const void* wscales, void* out,
                         hipStream_t st);
bool gemm_int4_fp6_init();
void launch_gemm_int4_fp6(const PrepackedGemmArgs& a, hipStream_t st);

}  // namespace svdq

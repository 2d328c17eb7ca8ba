// lora.hip -- a LoRA adapter merged into the SVDQuant low-rank branch.
//
// The low-rank branch is a 16-bit rank-r correction that runs beside the 4-bit product,
// and the modules keep their structure, so LoRA adapters keep working (page "Diffusers
// integra Nunchaku ...", "Nunchaku Lite: integración y modelo de ejecución"; page
// "Diffusers Natively Integrates Nunchaku Lite ...", the paragraph on loading through
// from_pretrained()).  An adapter y += alpha (x A^T) B^T, A [rl, K], B [N, rl], is the same
// kind of term as the branch's lora_act . l2^T with lora_act = x . l1^T, so it merges
// into the branch by concatenation:
//   l1' = [l1; A; 0]           [r', K]
//   l2' = [l2 | bf16(alpha B) | 0]   [N, r']
// with r' = r + rl rounded up to a multiple of 16 (the kernels' rank granularity; the
// zero rows and columns add exact zeros), and alpha B formed as one fp32 product rounded
// to bf16.  The activation kernel and the GEMM then run unchanged at rank r'.
#include "common.hpp"
#include "launch.hpp"

namespace svdq {
namespace {

__global__ __launch_bounds__(256) void merge_lora_kernel(int K, int N, int r, int rl, int ro,
                                                         const uint16_t* __restrict__ l1,
                                                         const uint16_t* __restrict__ l2,
                                                         const uint16_t* __restrict__ down,
                                                         const uint16_t* __restrict__ up, float alpha,
                                                         uint16_t* __restrict__ l1o,
                                                         uint16_t* __restrict__ l2o) {
    const int64_t n1 = (int64_t)ro * K, total = n1 + (int64_t)N * ro;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        if (i < n1) {
            const int row = (int)(i / K);
            const int64_t k = i - (int64_t)row * K;
            l1o[i] = row < r ? l1[(int64_t)row * K + k] : row < r + rl ? down[(int64_t)(row - r) * K + k] : (uint16_t)0;
        } else {
            const int64_t j2 = i - n1;
            const int64_t n = j2 / ro;
            const int j = (int)(j2 - n * ro);
            uint16_t v = 0;
            if (j < r) v = l2[n * r + j];
            else if (j < r + rl) v = (uint16_t)f32_to_bf16(alpha * bf16_to_f32(up[n * rl + (j - r)]));
            l2o[j2] = v;
        }
    }
}

}  // namespace

void launch_merge_lora(int K, int N, int r, int rl, int ro, const void* l1, const void* l2,
                       const void* down, const void* up, float alpha, void* l1o, void* l2o,
                       hipStream_t st) {
    const int64_t total = (int64_t)ro * K + (int64_t)N * ro;
    const int64_t blocks = std::min<int64_t>((total + 255) / 256, 4096);
    hipLaunchKernelGGL(merge_lora_kernel, dim3((unsigned)blocks), dim3(256), 0, st, K, N, r, rl, ro,
                       (const uint16_t*)l1, (const uint16_t*)l2, (const uint16_t*)down,
                       (const uint16_t*)up, alpha, (uint16_t*)l1o, (uint16_t*)l2o);
}

}  // namespace svdq

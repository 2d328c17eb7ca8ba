// host_driver.cpp -- calls every entry point of libsvdq's C ABI with argument sets that the
// validation must reject (null, misaligned or out-of-range values, bad enums, mismatched
// layer configurations), plus the pure size queries, for a build whose host code carries
// -fsanitize=address,undefined.  No call reaches a launch, so it runs on hosts without a GPU
// (and on hosts with one).  Exits non-zero if a call that must fail returns SVDQ_OK.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/svdq.h"
#include "../../include/svdq_peaks.h"

static int failures = 0;
#define MUST_FAIL(expr)                                                               \
    do {                                                                              \
        if ((expr) == SVDQ_OK) {                                                      \
            std::printf("accepted: %s\n", #expr);                                     \
            ++failures;                                                               \
        } else if (std::strlen(svdq_last_error()) == 0) {                             \
            std::printf("no message: %s\n", #expr);                                   \
            ++failures;                                                               \
        }                                                                             \
    } while (0)

int main() {
    void* F = reinterpret_cast<void*>(uintptr_t(1) << 20);   // aligned, never dereferenced
    void* Fm = reinterpret_cast<void*>((uintptr_t(1) << 20) + 2);
    svdq_stream_t st = nullptr;
    svdq_layer_cfg ok{3072, 3072, 32, 64, SVDQ_PREC_INT4};
    svdq_layer_cfg nv{3072, 9216, 32, 16, SVDQ_PREC_NVFP4};
    svdq_layer_cfg bad_k{100, 64, 16, 64, SVDQ_PREC_INT4};
    svdq_layer_cfg bad_r{512, 64, 20, 64, SVDQ_PREC_INT4};
    svdq_layer_cfg big_r{512, 64, 144, 64, SVDQ_PREC_INT4};
    svdq_layer_cfg bad_g{512, 64, 16, 32, SVDQ_PREC_INT4};
    svdq_layer_cfg bad_p{512, 64, 16, 64, 7};
    const svdq_layer_cfg* cfgs[] = {nullptr, &bad_k, &bad_r, &big_r, &bad_g, &bad_p};
    for (const svdq_layer_cfg* c : cfgs) {
        MUST_FAIL(svdq_quantize_act(c, 16, F, (const float*)F, F, 1.0f, F, F, F, st));
        MUST_FAIL(svdq_gemm_w4a4(c, 16, F, F, 1.0f, F, F, 1.0f, F, F, nullptr, 0, 0, F, st));
        MUST_FAIL(svdq_gemm_w4a4_packed(c, 16, F, F, F, F, nullptr, 0, 0, F, st));
        MUST_FAIL(svdq_gemm_w4a4_packed_noalloc(c, 16, F, F, F, F, nullptr, 0, 0, F, st));
        MUST_FAIL(svdq_quantize_act_packed(c, 16, F, (const float*)F, F, F, (float*)F, F, st));
    }
    MUST_FAIL(svdq_quantize_act(&ok, -1, F, (const float*)F, F, 1.0f, F, F, F, st));
    MUST_FAIL(svdq_quantize_act(&ok, 16, Fm, (const float*)F, F, 1.0f, F, F, F, st));
    MUST_FAIL(svdq_quantize_act(&nv, 16, F, (const float*)F, F, -1.0f, F, F, F, st));
    MUST_FAIL(svdq_quantize_act(&ok, 16, F, (const float*)F, nullptr, 1.0f, F, F, F, st));
    MUST_FAIL(svdq_gemm_w4a4(&ok, 16, F, F, 1.0f, F, F, 1.0f, F, F, Fm, 0, 0, F, st));
    MUST_FAIL(svdq_gemm_w4a4(&ok, 16, F, F, 1.0f, F, F, 1.0f, F, F, nullptr, 5, 0, F, st));
    MUST_FAIL(svdq_gemm_w4a4(&ok, 16, F, F, 1.0f, F, F, 1.0f, F, F, nullptr, 0, 9, F, st));
    MUST_FAIL(svdq_gemm_w4a4(&nv, 16, F, F, 0.0f, F, F, 1.0f, F, F, nullptr, 0, 0, F, st));
    MUST_FAIL(awq_gemm_w4a16(2, 100, 64, 64, F, F, F, F, nullptr, 0, F, st));
    MUST_FAIL(awq_gemm_w4a16(2, 128, 64, 32, F, F, F, F, nullptr, 0, F, st));
    MUST_FAIL(awq_gemm_w4a16(2, 128, 64, 64, Fm, F, F, F, nullptr, 0, F, st));
    MUST_FAIL(awq_gemm_w4a16(-3, 128, 64, 64, F, F, F, F, nullptr, 0, F, st));
    int64_t n = 0;
    MUST_FAIL(svdq_act_packed_bytes(&nv, 16, &n));
    MUST_FAIL(svdq_act_packed_bytes(&ok, -1, &n));
    MUST_FAIL(svdq_prepacked_weight_bytes(&ok, nullptr));
    MUST_FAIL(svdq_prepacked_l1_bytes(&nv, &n));
    MUST_FAIL(svdq_prepack_l1(&ok, nullptr, F, st));
    MUST_FAIL(svdq_pack_act(&ok, 16, F, (const float*)Fm, F, st));
    MUST_FAIL(svdq_prepack_weight(&ok, F, F, Fm, st));
    MUST_FAIL(svdq_gemm_w4a4_packed(&ok, 16, F, F, F, F, Fm, 0, 0, F, st));
    MUST_FAIL(svdq_gemm_w4a4_packed_workspace_bytes(&ok, -1, 0, 0, &n));
    MUST_FAIL(svdq_gemm_w4a4_packed_workspace_bytes(&ok, 16, 3, 0, &n));
    MUST_FAIL(svdq_gemm_w4a4_packed_ws(&ok, 16, F, F, F, F, nullptr, 0, 0, F, nullptr, 1024, st));
    MUST_FAIL(svdq_gemm_w4a4_packed_ws(&ok, 16, F, F, F, F, nullptr, 0, 0, F, Fm, 1024, st));
    MUST_FAIL(svdq_gemm_w4a4_packed_ws(&ok, 16, F, F, F, F, nullptr, 0, 0, F, F, -16, st));
    svdq_layer_cfg next_bad{1024, 3072, 32, 64, SVDQ_PREC_INT4};
    MUST_FAIL(svdq_quantize_next_workspace_bytes(&ok, &nv, 16, &n));
    MUST_FAIL(svdq_gemm_w4a4_packed_quantize_next(&ok, 16, F, F, F, F, nullptr, 1, &next_bad,
                                                  (const float*)F, F, F, nullptr, F, (float*)F, st));
    MUST_FAIL(svdq_calib_absmax(10, 100, F, (float*)F, st));
    MUST_FAIL(svdq_smoothing_factors(&ok, (const float*)F, (const float*)F, nullptr, (float*)F, st));
    MUST_FAIL(svdq_quantize_residual(&nv, (const float*)F, (const float*)F, F, F, F, F, nullptr, st));
    MUST_FAIL(svdq_lowrank_factors(&ok, (const float*)F, (const float*)F, (const float*)F, 16, 2, F,
                                   F, nullptr, F, st));
    MUST_FAIL(svdq_lowrank_factors(&big_r, (const float*)F, (const float*)F, (const float*)F, 64, 2, F,
                                   F, nullptr, F, st));
    MUST_FAIL(svdq_merge_lora(&ok, 0, F, F, F, F, 1.0f, F, F, st));
    MUST_FAIL(svdq_merge_lora(&ok, 120, F, F, F, F, 1.0f, F, F, st));
    MUST_FAIL(svdq_peak_mfma(9, 16, (float*)F, &n, st));
    MUST_FAIL(svdq_peak_copy(F, F, 4096, st));       // overlapping
    MUST_FAIL(svdq_peak_read(F, 100, F, st));
    MUST_FAIL(svdq_check_arch(nullptr));
    MUST_FAIL(svdq_check_arch("gfx942"));
    MUST_FAIL(svdq_check_device(-1));
    // size queries that need no device
    if (svdq_quantize_next_workspace_bytes(&ok, &ok, 300, &n) != SVDQ_OK || n != 16 * 512 * 32 * 4) ++failures;
    if (svdq_prepacked_l1_bytes(&ok, &n) != SVDQ_OK || n != 3072 * 32 * 2) ++failures;
    if (svdq_merged_rank(32, 16) != 48 || svdq_merged_rank(-1, 2) != -1) ++failures;
    for (int s = -1; s < 7; ++s)
        if (svdq_status_string((svdq_status)s) == nullptr) ++failures;
    std::printf("host driver: %d failures, version %d\n", failures, svdq_version());
    return failures == 0 ? 0 : 1;
}

// api.hip -- the extern "C" boundary of libsvdq: argument validation, the device
// capability check and dispatch to the gfx950 kernels.  Declarations and the contract of
// every entry point are in include/svdq.h.
//
// The capability check follows the pages' rule that an unsupported GPU must fail loudly
// and never return wrong results (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
// Diffusers", 技术细节 3; page "Nunchaku Lite: 4-битная генерация ...", "Какое железо и
// модели поддержаны"): every compute entry point checks that the current device is gfx950.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include <hip/hip_runtime.h>

#include "../../include/svdq.h"
#include "../../include/svdq_peaks.h"
#include "launch.hpp"
#include "packed_layout.hpp"

namespace {

thread_local std::string g_last_error;

svdq_status fail(svdq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
svdq_status fail(svdq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_state[kMaxDevices];   // 0 unknown, 1 gfx950, 2 other

bool arch_is_gfx950(const char* name) {
    return std::strncmp(name, "gfx950", 6) == 0 && (name[6] == '\0' || name[6] == ':');
}

svdq_status check_device_ordinal(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return fail(SVDQ_ERR_INVALID_ARG, "device ordinal %d out of range", dev);
    int s = g_dev_state[dev].load(std::memory_order_relaxed);
    if (s == 0) {
        hipDeviceProp_t prop;
        hipError_t e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(SVDQ_ERR_INVALID_ARG, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
        s = arch_is_gfx950(prop.gcnArchName) ? 1 : 2;
        g_dev_state[dev].store(s, std::memory_order_relaxed);
        if (s == 2)
            return fail(SVDQ_ERR_UNSUPPORTED_DEVICE,
                        "device %d is %s; this library's 4-bit kernels are built for gfx950 only",
                        dev, prop.gcnArchName);
    }
    if (s == 2)
        return fail(SVDQ_ERR_UNSUPPORTED_DEVICE,
                    "device %d is not gfx950; this library's 4-bit kernels are built for gfx950 only",
                    dev);
    return SVDQ_OK;
}

svdq_status check_current_device() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "no HIP device: %s", hipGetErrorString(e));
    return check_device_ordinal(dev);
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

svdq_status check_ptr(const void* p, const char* name, size_t align) {
    if (p == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, align)) return fail(SVDQ_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
    return SVDQ_OK;
}

svdq_status check_cfg(const svdq_layer_cfg* cfg) {
    if (cfg == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "cfg is NULL");
    if (cfg->precision != SVDQ_PREC_INT4 && cfg->precision != SVDQ_PREC_NVFP4)
        return fail(SVDQ_ERR_INVALID_ARG, "precision %d is neither INT4 (0) nor NVFP4 (1)", cfg->precision);
    if (cfg->in_features <= 0 || cfg->in_features % 64 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "in_features %d must be a positive multiple of 64", cfg->in_features);
    if (cfg->out_features <= 0)
        return fail(SVDQ_ERR_INVALID_ARG, "out_features %d must be positive", cfg->out_features);
    const int want_g = cfg->precision == SVDQ_PREC_INT4 ? 64 : 16;
    if (cfg->group_size != want_g)
        return fail(SVDQ_ERR_INVALID_ARG, "group_size %d: %s requires %d", cfg->group_size,
                    cfg->precision == SVDQ_PREC_INT4 ? "INT4" : "NVFP4", want_g);
    if (cfg->rank < 0 || cfg->rank % 16 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "rank %d must be 0 or a positive multiple of 16", cfg->rank);
    if (cfg->rank > 128)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "rank %d exceeds the supported maximum 128", cfg->rank);
    return SVDQ_OK;
}

svdq_status check_int4(const svdq_layer_cfg* cfg) {
    if (cfg->precision != SVDQ_PREC_INT4)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "packed operands exist for INT4 only");
    return SVDQ_OK;
}

svdq_status check_global_scale(float s, const char* name) {
    if (!(std::isfinite(s) && s > 0.0f))
        return fail(SVDQ_ERR_INVALID_ARG, "%s = %g must be finite and positive", name, (double)s);
    return SVDQ_OK;
}

svdq_status after_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(SVDQ_ERR_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
    return SVDQ_OK;
}

#define SVDQ_TRY(expr)                     \
    do {                                   \
        svdq_status _s = (expr);           \
        if (_s != SVDQ_OK) return _s;      \
    } while (0)

}  // namespace

extern "C" {

svdq_status svdq_quantize_act(const svdq_layer_cfg* cfg, int64_t M, const void* x,
                              const float* smooth_inv, const void* l1, float act_global_scale,
                              void* act_codes, void* act_scales, void* lora_act,
                              svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    const bool nvfp4 = cfg->precision == SVDQ_PREC_NVFP4;
    SVDQ_TRY(check_ptr(x, "x", 16));
    SVDQ_TRY(check_ptr(smooth_inv, "smooth_inv", 16));
    SVDQ_TRY(check_ptr(act_codes, "act_codes", 16));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", nvfp4 ? 1 : 4));
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(l1, "l1", 16));
        SVDQ_TRY(check_ptr(lora_act, "lora_act", 16));
    }
    if (nvfp4) SVDQ_TRY(check_global_scale(act_global_scale, "act_global_scale"));
    if (M > (int64_t)1 << 35)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::QuantArgs a{M, cfg->in_features, cfg->rank, nvfp4 ? 2 : 0, x, smooth_inv, l1,
                      act_global_scale, act_codes, act_scales, lora_act};
    svdq::launch_quantize_act(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_quantize_act");
}

svdq_status svdq_gemm_w4a4(const svdq_layer_cfg* cfg, int64_t M, const void* act_codes,
                           const void* act_scales, float act_global_scale, const void* wgt_codes,
                           const void* wgt_scales, float wgt_global_scale, const void* lora_act,
                           const void* l2, const void* bias, int32_t act, int32_t out_dtype,
                           void* out, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    const bool nvfp4 = cfg->precision == SVDQ_PREC_NVFP4;
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_INVALID_ARG, "act %d is not a svdq_act value", act);
    if (out_dtype != SVDQ_DT_F32 && out_dtype != SVDQ_DT_BF16)
        return fail(SVDQ_ERR_INVALID_ARG, "out_dtype %d is not a svdq_dtype value", out_dtype);
    SVDQ_TRY(check_ptr(act_codes, "act_codes", 16));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", nvfp4 ? 1 : 4));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", 16));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", nvfp4 ? 1 : 4));
    SVDQ_TRY(check_ptr(out, "out", out_dtype == SVDQ_DT_F32 ? 4 : 2));
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(lora_act, "lora_act", 16));
        SVDQ_TRY(check_ptr(l2, "l2", 16));
    }
    if (bias != nullptr && !aligned(bias, 2)) return fail(SVDQ_ERR_INVALID_ARG, "bias is not 2-byte aligned");
    if (nvfp4) {
        SVDQ_TRY(check_global_scale(act_global_scale, "act_global_scale"));
        SVDQ_TRY(check_global_scale(wgt_global_scale, "wgt_global_scale"));
    }
    if ((M + 127) / 128 > 65535)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::GemmArgs a{M, cfg->out_features, cfg->in_features, cfg->rank, nvfp4, act_codes, act_scales,
                     act_global_scale, wgt_codes, wgt_scales, wgt_global_scale, lora_act, l2, bias,
                     act, out_dtype == SVDQ_DT_BF16 ? 1 : 0, out};
    if (nvfp4) svdq::launch_gemm_nvfp4(a, reinterpret_cast<hipStream_t>(stream));
    else svdq::launch_gemm_int4(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_gemm_w4a4");
}

svdq_status awq_gemm_w4a16(int64_t M, int32_t K, int32_t N, int32_t group_size, const void* x,
                           const void* qweight, const void* scales, const void* zeros,
                           const void* bias, int32_t out_dtype, void* out, svdq_stream_t stream) {
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (K <= 0 || K % 64 != 0) return fail(SVDQ_ERR_INVALID_ARG, "K %d must be a positive multiple of 64", K);
    if (N <= 0) return fail(SVDQ_ERR_INVALID_ARG, "N %d must be positive", N);
    if (group_size != 64) return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "group_size %d: only 64 is supported", group_size);
    if (out_dtype != SVDQ_DT_F32 && out_dtype != SVDQ_DT_BF16)
        return fail(SVDQ_ERR_INVALID_ARG, "out_dtype %d is not a svdq_dtype value", out_dtype);
    SVDQ_TRY(check_ptr(x, "x", 16));
    SVDQ_TRY(check_ptr(qweight, "qweight", 16));
    SVDQ_TRY(check_ptr(scales, "scales", 2));
    SVDQ_TRY(check_ptr(zeros, "zeros", 2));
    SVDQ_TRY(check_ptr(out, "out", out_dtype == SVDQ_DT_F32 ? 4 : 2));
    if (bias != nullptr && !aligned(bias, 2)) return fail(SVDQ_ERR_INVALID_ARG, "bias is not 2-byte aligned");
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::AwqArgs a{M, K, N, x, qweight, scales, zeros, bias, out_dtype == SVDQ_DT_BF16 ? 1 : 0, out};
    svdq::launch_awq_gemv(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch("awq_gemm_w4a16");
}

svdq_status svdq_act_packed_bytes(const svdq_layer_cfg* cfg, int64_t M, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    *bytes = svdq::packed::act_bytes(M, cfg->in_features);
    return SVDQ_OK;
}

svdq_status svdq_prepacked_weight_bytes(const svdq_layer_cfg* cfg, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = svdq::packed::wgt_bytes(cfg->out_features, cfg->in_features);
    return SVDQ_OK;
}

svdq_status svdq_merge_lora(const svdq_layer_cfg* cfg, int32_t r_lora, const void* l1,
                            const void* l2, const void* lora_down, const void* lora_up,
                            float alpha, void* l1_out, void* l2_out, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    if (r_lora <= 0) return fail(SVDQ_ERR_INVALID_ARG, "r_lora = %d must be positive", r_lora);
    const int ro = svdq_merged_rank(cfg->rank, r_lora);
    if (ro > 128)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "merged rank %d exceeds the supported maximum 128", ro);
    if (!std::isfinite(alpha)) return fail(SVDQ_ERR_INVALID_ARG, "alpha is not finite");
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(l1, "l1", 2));
        SVDQ_TRY(check_ptr(l2, "l2", 2));
    }
    SVDQ_TRY(check_ptr(lora_down, "lora_down", 2));
    SVDQ_TRY(check_ptr(lora_up, "lora_up", 2));
    SVDQ_TRY(check_ptr(l1_out, "l1_out", 2));
    SVDQ_TRY(check_ptr(l2_out, "l2_out", 2));
    SVDQ_TRY(check_current_device());
    svdq::launch_merge_lora(cfg->in_features, cfg->out_features, cfg->rank, r_lora, ro, l1, l2,
                            lora_down, lora_up, alpha, l1_out, l2_out,
                            reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_merge_lora");
}

int32_t svdq_merged_rank(int32_t rank, int32_t r_lora) {
    if (rank < 0 || r_lora < 0) return -1;
    return (rank + r_lora + 15) / 16 * 16;
}

svdq_status svdq_prepacked_l1_bytes(const svdq_layer_cfg* cfg, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = svdq::prepacked_l1_bytes(cfg->rank, cfg->in_features);
    return SVDQ_OK;
}

svdq_status svdq_prepack_l1(const svdq_layer_cfg* cfg, const void* l1, void* l1_packed,
                            svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (cfg->rank == 0) return SVDQ_OK;
    SVDQ_TRY(check_ptr(l1, "l1", 16));
    SVDQ_TRY(check_ptr(l1_packed, "l1_packed", 16));
    SVDQ_TRY(check_current_device());
    svdq::launch_prepack_l1(cfg->rank, cfg->in_features, l1, l1_packed,
                            reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_prepack_l1");
}

svdq_status svdq_quantize_act_packed(const svdq_layer_cfg* cfg, int64_t M, const void* x,
                                     const float* smooth_inv, const void* l1_packed,
                                     void* act_packed, float* act_scales, void* lora_act,
                                     svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    SVDQ_TRY(check_ptr(x, "x", 16));
    SVDQ_TRY(check_ptr(smooth_inv, "smooth_inv", 16));
    SVDQ_TRY(check_ptr(act_packed, "act_packed", 16));
    if (act_scales != nullptr && !aligned(act_scales, 4))
        return fail(SVDQ_ERR_INVALID_ARG, "act_scales is not 4-byte aligned");
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(l1_packed, "l1_packed", 16));
        SVDQ_TRY(check_ptr(lora_act, "lora_act", 16));
    }
    if (M > (int64_t)1 << 35)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::QuantArgs a{M, cfg->in_features, cfg->rank, 1, x, smooth_inv, l1_packed, 1.0f, act_packed,
                      act_scales, lora_act};
    svdq::launch_quantize_act(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_quantize_act_packed");
}

svdq_status svdq_pack_act(const svdq_layer_cfg* cfg, int64_t M, const void* act_codes,
                          const float* act_scales, void* act_packed, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    SVDQ_TRY(check_ptr(act_codes, "act_codes", 16));
    SVDQ_TRY(check_ptr(act_scales, "act_scales", 4));
    SVDQ_TRY(check_ptr(act_packed, "act_packed", 16));
    const int64_t blocks = (M + 255) / 256 * 8 * (int64_t)(cfg->in_features / 64);
    if (blocks >= (int64_t)1 << 31)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::launch_pack_act(M, cfg->in_features, act_codes, act_scales, act_packed,
                          reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_pack_act");
}

svdq_status svdq_prepack_weight(const svdq_layer_cfg* cfg, const void* wgt_codes,
                                const void* wgt_scales, void* prepacked, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", 16));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", 4));
    SVDQ_TRY(check_ptr(prepacked, "prepacked", 16));
    const int64_t blocks = (int64_t)(cfg->out_features + 191) / 192 * 6 * (cfg->in_features / 64);
    if (blocks >= (int64_t)1 << 31)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "layer too large for one launch");
    SVDQ_TRY(check_current_device());
    svdq::launch_prepack_wgt(cfg->out_features, cfg->in_features, wgt_codes, wgt_scales, prepacked,
                             reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_prepack_weight");
}

}  // extern "C"

namespace {

// Shared body of the packed GEMM entry points: validation, then the launch with the K-split
// workspace `ws` of `ws_bytes` bytes (NULL: no K split).
svdq_status gemm_packed(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                        const void* prepacked, const void* lora_act, const void* l2,
                        const void* bias, int32_t act, int32_t out_dtype, void* out, void* ws,
                        int64_t ws_bytes, svdq_stream_t stream, const char* name) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_INVALID_ARG, "act %d is not a svdq_act value", act);
    if (out_dtype != SVDQ_DT_F32 && out_dtype != SVDQ_DT_BF16)
        return fail(SVDQ_ERR_INVALID_ARG, "out_dtype %d is not a svdq_dtype value", out_dtype);
    SVDQ_TRY(check_ptr(act_packed, "act_packed", 16));
    SVDQ_TRY(check_ptr(prepacked, "prepacked", 16));
    SVDQ_TRY(check_ptr(out, "out", out_dtype == SVDQ_DT_F32 ? 4 : 2));
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(lora_act, "lora_act", 16));
        SVDQ_TRY(check_ptr(l2, "l2", 16));
    }
    if (bias != nullptr && !aligned(bias, 2)) return fail(SVDQ_ERR_INVALID_ARG, "bias is not 2-byte aligned");
    if (ws_bytes < 0) return fail(SVDQ_ERR_INVALID_ARG, "workspace_bytes = %lld is negative", (long long)ws_bytes);
    if (ws != nullptr && !aligned(ws, 16)) return fail(SVDQ_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
    const int64_t tiles = ((M + 255) / 256) * ((cfg->out_features + 191) / 192);
    if (tiles >= (int64_t)1 << 31)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    if (!svdq::gemm_w4a4_fp6_init())
        return fail(SVDQ_ERR_LAUNCH, "could not reserve LDS for the packed GEMM");
    svdq::PackedGemmArgs a{M, cfg->out_features, cfg->in_features, cfg->rank, act_packed,
                           prepacked, lora_act, l2, bias, act, out_dtype == SVDQ_DT_BF16 ? 1 : 0, out, 0};
    a.split_ws = ws_bytes > 0 ? static_cast<float*>(ws) : nullptr;
    a.split_ws_bytes = ws_bytes;
    svdq::launch_gemm_w4a4_fp6(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch(name);
}

}  // namespace

extern "C" {

svdq_status svdq_gemm_w4a4_packed(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                  const void* prepacked, const void* lora_act, const void* l2,
                                  const void* bias, int32_t act, int32_t out_dtype, void* out,
                                  svdq_stream_t stream) {
    return gemm_packed(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype, out,
                       nullptr, 0, stream, "svdq_gemm_w4a4_packed");
}

svdq_status svdq_gemm_w4a4_packed_workspace_bytes(const svdq_layer_cfg* cfg, int64_t M, int32_t act,
                                                  int32_t out_dtype, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_INVALID_ARG, "act %d is not a svdq_act value", act);
    if (out_dtype != SVDQ_DT_F32 && out_dtype != SVDQ_DT_BF16)
        return fail(SVDQ_ERR_INVALID_ARG, "out_dtype %d is not a svdq_dtype value", out_dtype);
    SVDQ_TRY(check_current_device());
    *bytes = M == 0 ? 0
                    : svdq::split_workspace_bytes(M, cfg->out_features, cfg->in_features, act,
                                                  out_dtype == SVDQ_DT_BF16 ? 1 : 0);
    return SVDQ_OK;
}

svdq_status svdq_gemm_w4a4_packed_ws(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                     const void* prepacked, const void* lora_act, const void* l2,
                                     const void* bias, int32_t act, int32_t out_dtype, void* out,
                                     void* workspace, int64_t workspace_bytes, svdq_stream_t stream) {
    if (workspace == nullptr && workspace_bytes > 0)
        return fail(SVDQ_ERR_INVALID_ARG, "workspace is NULL but workspace_bytes = %lld",
                    (long long)workspace_bytes);
    return gemm_packed(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype, out,
                       workspace, workspace_bytes, stream, "svdq_gemm_w4a4_packed_ws");
}

svdq_status svdq_gemm_w4a4_packed_noalloc(const svdq_layer_cfg* cfg, int64_t M, const void* act_packed,
                                          const void* prepacked, const void* lora_act, const void* l2,
                                          const void* bias, int32_t act, int32_t out_dtype, void* out,
                                          svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_INVALID_ARG, "act %d is not a svdq_act value", act);
    if (out_dtype != SVDQ_DT_F32 && out_dtype != SVDQ_DT_BF16)
        return fail(SVDQ_ERR_INVALID_ARG, "out_dtype %d is not a svdq_dtype value", out_dtype);
    SVDQ_TRY(check_current_device());
    void* ws = nullptr;
    int64_t ws_bytes = 0;
    const hipError_t e = svdq::noalloc_scratch(&ws, &ws_bytes);
    if (e != hipSuccess)
        return fail(SVDQ_ERR_LAUNCH, "device scratch of svdq_gemm_w4a4_packed_noalloc not found: %s",
                    hipGetErrorString(e));
    const int64_t need = M == 0 ? 0
                                : svdq::split_workspace_bytes(M, cfg->out_features, cfg->in_features, act,
                                                              out_dtype == SVDQ_DT_BF16 ? 1 : 0);
    if (need > ws_bytes)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG,
                    "the K split needs %lld bytes of scratch, more than the %lld the library holds",
                    (long long)need, (long long)ws_bytes);
    return gemm_packed(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype, out, ws,
                       need, stream, "svdq_gemm_w4a4_packed_noalloc");
}

svdq_status svdq_quantize_next_workspace_bytes(const svdq_layer_cfg* cfg, const svdq_layer_cfg* next_cfg,
                                               int64_t M, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    SVDQ_TRY(check_cfg(next_cfg));
    SVDQ_TRY(check_int4(next_cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    *bytes = svdq::quantize_next_workspace_bytes(M, cfg->out_features, next_cfg->rank);
    return SVDQ_OK;
}

svdq_status svdq_gemm_w4a4_packed_quantize_next(
    const svdq_layer_cfg* cfg, int64_t M, const void* act_packed, const void* prepacked,
    const void* lora_act, const void* l2, const void* bias, int32_t act,
    const svdq_layer_cfg* next_cfg, const float* next_smooth_inv, const void* next_l1,
    void* next_act_packed, float* next_act_scales, void* next_lora_act, float* lora_workspace,
    svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_int4(cfg));
    SVDQ_TRY(check_cfg(next_cfg));
    SVDQ_TRY(check_int4(next_cfg));
    if (next_cfg->in_features != cfg->out_features)
        return fail(SVDQ_ERR_INVALID_ARG, "next layer in_features %d != this layer's out_features %d",
                    next_cfg->in_features, cfg->out_features);
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (act != SVDQ_ACT_NONE && act != SVDQ_ACT_GELU_TANH)
        return fail(SVDQ_ERR_INVALID_ARG, "act %d is not a svdq_act value", act);
    SVDQ_TRY(check_ptr(act_packed, "act_packed", 16));
    SVDQ_TRY(check_ptr(prepacked, "prepacked", 16));
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(lora_act, "lora_act", 16));
        SVDQ_TRY(check_ptr(l2, "l2", 16));
    }
    if (bias != nullptr && !aligned(bias, 2)) return fail(SVDQ_ERR_INVALID_ARG, "bias is not 2-byte aligned");
    SVDQ_TRY(check_ptr(next_smooth_inv, "next_smooth_inv", 16));
    SVDQ_TRY(check_ptr(next_act_packed, "next_act_packed", 16));
    if (next_act_scales != nullptr && !aligned(next_act_scales, 4))
        return fail(SVDQ_ERR_INVALID_ARG, "next_act_scales is not 4-byte aligned");
    if (next_cfg->rank > 0) {
        SVDQ_TRY(check_ptr(next_l1, "next_l1", 16));
        SVDQ_TRY(check_ptr(next_lora_act, "next_lora_act", 8));
        SVDQ_TRY(check_ptr(lora_workspace, "lora_workspace", 16));
    }
    const int64_t tiles = ((M + 255) / 256) * ((cfg->out_features + 191) / 192);
    if (tiles >= (int64_t)1 << 31)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    if (!svdq::gemm_w4a4_fp6_init())
        return fail(SVDQ_ERR_LAUNCH, "could not reserve LDS for the packed GEMM");
    svdq::PackedGemmArgs a{M, cfg->out_features, cfg->in_features, cfg->rank, act_packed,
                           prepacked, lora_act, l2, bias, act, 1, next_lora_act, 0};
    a.quantize_next = 1;
    a.next_r = next_cfg->rank;
    a.next_si = next_smooth_inv;
    a.next_l1 = next_l1;
    a.next_packed = next_act_packed;
    a.next_scales = next_act_scales;
    a.lora_work = lora_workspace;
    svdq::launch_gemm_w4a4_fp6(a, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_gemm_w4a4_packed_quantize_next");
}

svdq_status svdq_calib_absmax(int64_t M, int32_t K, const void* x, float* absmax,
                              svdq_stream_t stream) {
    if (M < 0) return fail(SVDQ_ERR_INVALID_ARG, "M = %lld is negative", (long long)M);
    if (K <= 0 || K % 64 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "K = %d must be a positive multiple of 64", K);
    if (M > 0) SVDQ_TRY(check_ptr(x, "x", 16));
    SVDQ_TRY(check_ptr(absmax, "absmax", 16));
    if ((M + 63) / 64 >= 65536)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "M = %lld too large for one launch", (long long)M);
    SVDQ_TRY(check_current_device());
    if (M == 0) return SVDQ_OK;
    svdq::launch_calib_absmax(M, K, x, absmax, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_calib_absmax");
}

svdq_status svdq_smoothing_factors(const svdq_layer_cfg* cfg, const float* w, const float* x_absmax,
                                   float* w_absmax, float* smooth_inv, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    SVDQ_TRY(check_ptr(w, "w", 16));
    SVDQ_TRY(check_ptr(x_absmax, "x_absmax", 4));
    SVDQ_TRY(check_ptr(w_absmax, "w_absmax", 16));
    SVDQ_TRY(check_ptr(smooth_inv, "smooth_inv", 4));
    if ((cfg->out_features + 31) / 32 >= 65536)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "out_features %d too large for one launch", cfg->out_features);
    SVDQ_TRY(check_current_device());
    svdq::launch_smoothing_factors(cfg->out_features, cfg->in_features, w, x_absmax, w_absmax,
                                   smooth_inv, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_smoothing_factors");
}

svdq_status svdq_quantize_residual(const svdq_layer_cfg* cfg, const float* w, const float* smooth_inv,
                                   const void* l1, const void* l2, void* wgt_codes, void* wgt_scales,
                                   float* wgt_global_scale, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    const bool nv = cfg->precision == SVDQ_PREC_NVFP4;
    SVDQ_TRY(check_ptr(w, "w", 16));
    SVDQ_TRY(check_ptr(smooth_inv, "smooth_inv", 16));
    if (cfg->rank > 0) {
        SVDQ_TRY(check_ptr(l1, "l1", 16));
        SVDQ_TRY(check_ptr(l2, "l2", 2));
    }
    SVDQ_TRY(check_ptr(wgt_codes, "wgt_codes", 16));
    SVDQ_TRY(check_ptr(wgt_scales, "wgt_scales", nv ? 2 : 4));
    if (nv) SVDQ_TRY(check_ptr(wgt_global_scale, "wgt_global_scale", 4));
    if ((int64_t)cfg->out_features * (cfg->in_features / 32) / 256 >= ((int64_t)1 << 31))
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "layer too large for one launch");
    SVDQ_TRY(check_current_device());
    svdq::launch_quantize_residual(cfg->out_features, cfg->in_features, cfg->rank, nv, w, smooth_inv,
                                   l1, l2, wgt_codes, wgt_scales, wgt_global_scale,
                                   reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_quantize_residual");
}

svdq_status svdq_lowrank_workspace_bytes(const svdq_layer_cfg* cfg, int64_t* bytes) {
    SVDQ_TRY(check_cfg(cfg));
    if (bytes == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = svdq::lowrank_workspace_bytes(cfg->out_features, cfg->in_features);
    return SVDQ_OK;
}

svdq_status svdq_lowrank_factors(const svdq_layer_cfg* cfg, const float* w, const float* smooth_inv,
                                 const float* omega, int32_t block, int32_t iters, void* l1, void* l2,
                                 float* sigma, void* workspace, svdq_stream_t stream) {
    SVDQ_TRY(check_cfg(cfg));
    const int r = cfg->rank;
    if (r <= 0 || r > 64)
        return fail(SVDQ_ERR_UNSUPPORTED_CONFIG, "rank %d: the factorization takes ranks 16 to 64", r);
    if (block < r || block > 64)
        return fail(SVDQ_ERR_INVALID_ARG, "block %d must lie in [rank %d, 64]", block, r);
    if (iters < 0 || iters > 32) return fail(SVDQ_ERR_INVALID_ARG, "iters %d must lie in [0, 32]", iters);
    SVDQ_TRY(check_ptr(w, "w", 4));
    SVDQ_TRY(check_ptr(smooth_inv, "smooth_inv", 4));
    SVDQ_TRY(check_ptr(omega, "omega", 4));
    SVDQ_TRY(check_ptr(l1, "l1", 2));
    SVDQ_TRY(check_ptr(l2, "l2", 2));
    if (sigma != nullptr && !aligned(sigma, 4)) return fail(SVDQ_ERR_INVALID_ARG, "sigma is not 4-byte aligned");
    SVDQ_TRY(check_ptr(workspace, "workspace", 16));
    SVDQ_TRY(check_current_device());
    svdq::launch_lowrank_factors(cfg->out_features, cfg->in_features, r, block, iters, w, smooth_inv, omega,
                                 l1, l2, sigma, workspace, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_lowrank_factors");
}

svdq_status svdq_peak_mfma(int32_t kind, int32_t iters, float* out, int64_t* ops,
                           svdq_stream_t stream) {
    if (kind < 0 || kind > 5) return fail(SVDQ_ERR_INVALID_ARG, "kind %d is not in [0, 5]", kind);
    if (iters < 1 || iters > (1 << 20)) return fail(SVDQ_ERR_INVALID_ARG, "iters %d not in [1, 2^20]", iters);
    SVDQ_TRY(check_ptr(out, "out", 4));
    if (ops == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "ops is NULL");
    SVDQ_TRY(check_current_device());
    *ops = svdq::launch_mfma_peak(kind, iters, out, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_peak_mfma");
}

svdq_status svdq_peak_copy(const void* src, void* dst, int64_t bytes, svdq_stream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "bytes = %lld must be a positive multiple of 16", (long long)bytes);
    SVDQ_TRY(check_ptr(src, "src", 16));
    SVDQ_TRY(check_ptr(dst, "dst", 16));
    const uintptr_t s = reinterpret_cast<uintptr_t>(src), d = reinterpret_cast<uintptr_t>(dst);
    if (s < d + (uintptr_t)bytes && d < s + (uintptr_t)bytes)
        return fail(SVDQ_ERR_INVALID_ARG, "src and dst overlap");
    SVDQ_TRY(check_current_device());
    svdq::launch_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_peak_copy");
}

svdq_status svdq_peak_read(const void* src, int64_t bytes, void* out, svdq_stream_t stream) {
    if (bytes <= 0 || bytes % 16 != 0)
        return fail(SVDQ_ERR_INVALID_ARG, "bytes = %lld must be a positive multiple of 16", (long long)bytes);
    SVDQ_TRY(check_ptr(src, "src", 16));
    SVDQ_TRY(check_ptr(out, "out", 4));
    SVDQ_TRY(check_current_device());
    svdq::launch_read(src, bytes, out, reinterpret_cast<hipStream_t>(stream));
    return after_launch("svdq_peak_read");
}

svdq_status svdq_check_device(int device) { return check_device_ordinal(device); }

svdq_status svdq_check_arch(const char* arch_name) {
    if (arch_name == nullptr) return fail(SVDQ_ERR_INVALID_ARG, "arch_name is NULL");
    if (!arch_is_gfx950(arch_name))
        return fail(SVDQ_ERR_UNSUPPORTED_DEVICE, "architecture %s is not gfx950", arch_name);
    return SVDQ_OK;
}

const char* svdq_status_string(svdq_status status) {
    // the caller may pass any 32-bit value: read it as an integer, not as the enum (a value
    // outside the enum's range may not be loaded as the enum type)
    int32_t s;
    std::memcpy(&s, &status, sizeof s);
    switch (s) {
        case SVDQ_OK: return "SVDQ_OK";
        case SVDQ_ERR_INVALID_ARG: return "SVDQ_ERR_INVALID_ARG: invalid argument";
        case SVDQ_ERR_UNSUPPORTED_DEVICE: return "SVDQ_ERR_UNSUPPORTED_DEVICE: device is not gfx950";
        case SVDQ_ERR_UNSUPPORTED_CONFIG: return "SVDQ_ERR_UNSUPPORTED_CONFIG: configuration not supported";
        case SVDQ_ERR_LAUNCH: return "SVDQ_ERR_LAUNCH: kernel launch failed";
    }
    return "unknown svdq_status";
}

const char* svdq_last_error(void) { return g_last_error.c_str(); }

int32_t svdq_version(void) { return 100; }

}  // extern "C"

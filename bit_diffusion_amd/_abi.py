"""ctypes view of include/svdq.h: constants, the layer-config struct and function signatures.

The shared library must have been built (``python -m bit_diffusion_amd.build``); loading
fails loudly otherwise -- there is no fallback implementation.
"""
import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libsvdq.so")

SVDQ_OK = 0
SVDQ_ERR_INVALID_ARG = 1
SVDQ_ERR_UNSUPPORTED_DEVICE = 2
SVDQ_ERR_UNSUPPORTED_CONFIG = 3
SVDQ_ERR_LAUNCH = 4
SVDQ_PREC_INT4 = 0
SVDQ_PREC_NVFP4 = 1
SVDQ_DT_F32 = 0
SVDQ_DT_BF16 = 1
SVDQ_ACT_NONE = 0
SVDQ_ACT_GELU_TANH = 1

# Every symbol include/*.h declares.
EXPORTS = ("svdq_quantize_act", "svdq_gemm_w4a4", "awq_gemm_w4a16", "svdq_check_device",
           "svdq_check_arch", "svdq_status_string", "svdq_last_error", "svdq_version",
           "svdq_act_packed_bytes", "svdq_prepacked_weight_bytes", "svdq_quantize_act_packed",
           "svdq_pack_act", "svdq_prepack_weight", "svdq_gemm_w4a4_packed",
           "svdq_prepacked_l1_bytes", "svdq_prepack_l1", "svdq_merged_rank", "svdq_merge_lora",
           "svdq_gemm_w4a4_packed_quantize_next", "svdq_calib_absmax", "svdq_smoothing_factors",
           "svdq_quantize_residual", "svdq_lowrank_workspace_bytes", "svdq_lowrank_factors",
           "svdq_gemm_w4a4_packed_workspace_bytes", "svdq_gemm_w4a4_packed_ws",
           "svdq_quantize_next_workspace_bytes", "svdq_peak_mfma", "svdq_peak_copy",
           "svdq_gemm_w4a4_packed_noalloc", "svdq_peak_read")


class LayerCfg(ctypes.Structure):
    """svdq_layer_cfg: the per-layer quantization fields (in/out features, rank, group size,
    precision)."""
    _fields_ = [("in_features", ctypes.c_int32), ("out_features", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("precision", ctypes.c_int32)]

    @classmethod
    def make(cls, K, N, rank, precision="int4"):
        p = SVDQ_PREC_INT4 if precision == "int4" else SVDQ_PREC_NVFP4
        return cls(int(K), int(N), int(rank), 64 if p == SVDQ_PREC_INT4 else 16, p)


class SvdqError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"svdq status {status}: {message}")
        self.status = status
        self.message = message


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m bit_diffusion_amd.build` "
                "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
        cfgp = ctypes.POINTER(LayerCfg)
        L.svdq_quantize_act.argtypes = [cfgp, I64, P, P, P, F, P, P, P, P]
        L.svdq_gemm_w4a4.argtypes = [cfgp, I64, P, P, F, P, P, F, P, P, P, I32, I32, P, P]
        L.awq_gemm_w4a16.argtypes = [I64, I32, I32, I32, P, P, P, P, P, I32, P, P]
        L.svdq_act_packed_bytes.argtypes = [cfgp, I64, ctypes.POINTER(ctypes.c_int64)]
        L.svdq_prepacked_weight_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_int64)]
        L.svdq_quantize_act_packed.argtypes = [cfgp, I64, P, P, P, P, P, P, P]
        L.svdq_pack_act.argtypes = [cfgp, I64, P, P, P, P]
        L.svdq_prepack_weight.argtypes = [cfgp, P, P, P, P]
        L.svdq_prepacked_l1_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_int64)]
        L.svdq_prepack_l1.argtypes = [cfgp, P, P, P]
        L.svdq_merged_rank.argtypes = [I32, I32]
        L.svdq_merged_rank.restype = I32
        L.svdq_merge_lora.argtypes = [cfgp, I32, P, P, P, P, F, P, P, P]
        L.svdq_gemm_w4a4_packed_quantize_next.argtypes = [cfgp, I64, P, P, P, P, P, I32, cfgp, P, P,
                                                           P, P, P, P, P]
        L.svdq_calib_absmax.argtypes = [I64, I32, P, P, P]
        L.svdq_smoothing_factors.argtypes = [cfgp, P, P, P, P, P]
        L.svdq_quantize_residual.argtypes = [cfgp, P, P, P, P, P, P, P, P]
        L.svdq_lowrank_workspace_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_int64)]
        L.svdq_lowrank_factors.argtypes = [cfgp, P, P, P, I32, I32, P, P, P, P, P]
        L.svdq_gemm_w4a4_packed.argtypes = [cfgp, I64, P, P, P, P, P, I32, I32, P, P]
        L.svdq_gemm_w4a4_packed_workspace_bytes.argtypes = [cfgp, I64, I32, I32,
                                                            ctypes.POINTER(ctypes.c_int64)]
        L.svdq_gemm_w4a4_packed_ws.argtypes = [cfgp, I64, P, P, P, P, P, I32, I32, P, P, I64, P]
        L.svdq_quantize_next_workspace_bytes.argtypes = [cfgp, cfgp, I64,
                                                         ctypes.POINTER(ctypes.c_int64)]
        L.svdq_gemm_w4a4_packed_noalloc.argtypes = [cfgp, I64, P, P, P, P, P, I32, I32, P, P]
        L.svdq_peak_mfma.argtypes = [I32, I32, P, ctypes.POINTER(ctypes.c_int64), P]
        L.svdq_peak_copy.argtypes = [P, P, I64, P]
        L.svdq_peak_read.argtypes = [P, I64, P, P]
        L.svdq_check_device.argtypes = [ctypes.c_int]
        L.svdq_check_arch.argtypes = [ctypes.c_char_p]
        L.svdq_status_string.argtypes = [ctypes.c_int]
        L.svdq_status_string.restype = ctypes.c_char_p
        L.svdq_last_error.argtypes = []
        L.svdq_last_error.restype = ctypes.c_char_p
        L.svdq_version.restype = ctypes.c_int32
        for name in ("svdq_quantize_act", "svdq_gemm_w4a4", "awq_gemm_w4a16",
                     "svdq_check_device", "svdq_check_arch", "svdq_act_packed_bytes",
                     "svdq_prepacked_weight_bytes", "svdq_quantize_act_packed", "svdq_pack_act",
                     "svdq_prepack_weight", "svdq_gemm_w4a4_packed", "svdq_prepacked_l1_bytes",
                     "svdq_prepack_l1", "svdq_merge_lora", "svdq_gemm_w4a4_packed_quantize_next",
                     "svdq_calib_absmax", "svdq_smoothing_factors", "svdq_quantize_residual",
                     "svdq_lowrank_workspace_bytes", "svdq_lowrank_factors",
                     "svdq_gemm_w4a4_packed_workspace_bytes", "svdq_gemm_w4a4_packed_ws",
                     "svdq_quantize_next_workspace_bytes", "svdq_peak_mfma", "svdq_peak_copy",
                     "svdq_gemm_w4a4_packed_noalloc", "svdq_peak_read"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib

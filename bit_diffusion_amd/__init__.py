"""bit_diffusion_amd -- MI355X (gfx950) SVDQuant W4A4 / AWQ W4A16 linear layers.

Thin Python binding of the C ABI in include/svdq.h (libsvdq.so, built in-tree by
``python -m bit_diffusion_amd.build``).  Functions keep the C names and argument order;
they only marshal arguments: torch tensors become device pointers, the stream defaults to
torch's current stream, and a non-OK status raises SvdqError with the library's message.
Every computation runs in the library's HIP kernels; there is no fallback path.
"""
import ctypes
import os

from . import _abi
from ._abi import (SVDQ_OK, SVDQ_ERR_INVALID_ARG, SVDQ_ERR_UNSUPPORTED_DEVICE,  # noqa: F401
                   SVDQ_ERR_UNSUPPORTED_CONFIG, SVDQ_ERR_LAUNCH, SVDQ_PREC_INT4, SVDQ_PREC_NVFP4,
                   SVDQ_DT_F32, SVDQ_DT_BF16, SVDQ_ACT_NONE, SVDQ_ACT_GELU_TANH, LayerCfg,
                   SvdqError, lib, LIB_PATH)

__all__ = [
    "svdq_quantize_act", "svdq_gemm_w4a4", "awq_gemm_w4a16", "svdq_check_device",
    "svdq_act_packed_bytes", "svdq_prepacked_weight_bytes", "svdq_quantize_act_packed",
    "svdq_pack_act", "svdq_prepack_weight", "svdq_gemm_w4a4_packed",
    "svdq_prepacked_l1_bytes", "svdq_prepack_l1", "svdq_merged_rank", "svdq_merge_lora",
    "svdq_gemm_w4a4_packed_quantize_next", "svdq_calib_absmax", "svdq_smoothing_factors",
    "svdq_quantize_residual", "svdq_lowrank_workspace_bytes", "svdq_lowrank_factors",
    "svdq_gemm_w4a4_packed_workspace_bytes", "svdq_gemm_w4a4_packed_ws",
    "svdq_quantize_next_workspace_bytes", "svdq_peak_mfma", "svdq_peak_copy",
    "svdq_gemm_w4a4_packed_noalloc", "svdq_peak_read",
    "svdq_check_arch", "svdq_status_string", "svdq_last_error", "svdq_version", "LayerCfg",
    "SvdqError", "lib", "LIB_PATH",
]


def _ptr(t):
    """Device/host address of a tensor (or an int address, or None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != SVDQ_OK:
        raise SvdqError(status, svdq_last_error())
    return status


def svdq_quantize_act(cfg, M, x, smooth_inv, l1, act_global_scale, act_codes, act_scales,
                      lora_act, stream=None):
    L = lib()
    return _check(L.svdq_quantize_act(ctypes.byref(cfg), int(M), _ptr(x), _ptr(smooth_inv),
                                      _ptr(l1), float(act_global_scale), _ptr(act_codes),
                                      _ptr(act_scales), _ptr(lora_act), _stream(stream)))


def svdq_gemm_w4a4(cfg, M, act_codes, act_scales, act_global_scale, wgt_codes, wgt_scales,
                   wgt_global_scale, lora_act, l2, bias, act, out_dtype, out, stream=None):
    L = lib()
    return _check(L.svdq_gemm_w4a4(ctypes.byref(cfg), int(M), _ptr(act_codes), _ptr(act_scales),
                                   float(act_global_scale), _ptr(wgt_codes), _ptr(wgt_scales),
                                   float(wgt_global_scale), _ptr(lora_act), _ptr(l2), _ptr(bias),
                                   int(act), int(out_dtype), _ptr(out), _stream(stream)))


def awq_gemm_w4a16(M, K, N, group_size, x, qweight, scales, zeros, bias, out_dtype, out,
                   stream=None):
    L = lib()
    return _check(L.awq_gemm_w4a16(int(M), int(K), int(N), int(group_size), _ptr(x),
                                   _ptr(qweight), _ptr(scales), _ptr(zeros), _ptr(bias),
                                   int(out_dtype), _ptr(out), _stream(stream)))


def svdq_act_packed_bytes(cfg, M):
    n = ctypes.c_int64(0)
    _check(lib().svdq_act_packed_bytes(ctypes.byref(cfg), int(M), ctypes.byref(n)))
    return n.value


def svdq_prepacked_weight_bytes(cfg):
    n = ctypes.c_int64(0)
    _check(lib().svdq_prepacked_weight_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def svdq_merged_rank(rank, r_lora):
    return int(lib().svdq_merged_rank(int(rank), int(r_lora)))


def svdq_merge_lora(cfg, r_lora, l1, l2, lora_down, lora_up, alpha, l1_out, l2_out, stream=None):
    return _check(lib().svdq_merge_lora(ctypes.byref(cfg), int(r_lora), _ptr(l1), _ptr(l2),
                                        _ptr(lora_down), _ptr(lora_up), float(alpha),
                                        _ptr(l1_out), _ptr(l2_out), _stream(stream)))


def svdq_prepacked_l1_bytes(cfg):
    n = ctypes.c_int64(0)
    _check(lib().svdq_prepacked_l1_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def svdq_prepack_l1(cfg, l1, l1_packed, stream=None):
    return _check(lib().svdq_prepack_l1(ctypes.byref(cfg), _ptr(l1), _ptr(l1_packed),
                                        _stream(stream)))


def svdq_quantize_act_packed(cfg, M, x, smooth_inv, l1_packed, act_packed, act_scales, lora_act,
                             stream=None):
    return _check(lib().svdq_quantize_act_packed(
        ctypes.byref(cfg), int(M), _ptr(x), _ptr(smooth_inv), _ptr(l1_packed), _ptr(act_packed),
        _ptr(act_scales), _ptr(lora_act), _stream(stream)))


def svdq_pack_act(cfg, M, act_codes, act_scales, act_packed, stream=None):
    return _check(lib().svdq_pack_act(ctypes.byref(cfg), int(M), _ptr(act_codes),
                                      _ptr(act_scales), _ptr(act_packed), _stream(stream)))


def svdq_prepack_weight(cfg, wgt_codes, wgt_scales, prepacked, stream=None):
    return _check(lib().svdq_prepack_weight(ctypes.byref(cfg), _ptr(wgt_codes), _ptr(wgt_scales),
                                            _ptr(prepacked), _stream(stream)))


def svdq_gemm_w4a4_packed(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype, out,
                          stream=None):
    return _check(lib().svdq_gemm_w4a4_packed(
        ctypes.byref(cfg), int(M), _ptr(act_packed), _ptr(prepacked), _ptr(lora_act), _ptr(l2),
        _ptr(bias), int(act), int(out_dtype), _ptr(out), _stream(stream)))


def svdq_gemm_w4a4_packed_workspace_bytes(cfg, M, act, out_dtype):
    n = ctypes.c_int64(0)
    _check(lib().svdq_gemm_w4a4_packed_workspace_bytes(ctypes.byref(cfg), int(M), int(act),
                                                       int(out_dtype), ctypes.byref(n)))
    return n.value


def svdq_gemm_w4a4_packed_ws(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype, out,
                             workspace, workspace_bytes, stream=None):
    return _check(lib().svdq_gemm_w4a4_packed_ws(
        ctypes.byref(cfg), int(M), _ptr(act_packed), _ptr(prepacked), _ptr(lora_act), _ptr(l2),
        _ptr(bias), int(act), int(out_dtype), _ptr(out), _ptr(workspace), int(workspace_bytes),
        _stream(stream)))


def svdq_gemm_w4a4_packed_noalloc(cfg, M, act_packed, prepacked, lora_act, l2, bias, act, out_dtype,
                                  out, stream=None):
    return _check(lib().svdq_gemm_w4a4_packed_noalloc(
        ctypes.byref(cfg), int(M), _ptr(act_packed), _ptr(prepacked), _ptr(lora_act), _ptr(l2),
        _ptr(bias), int(act), int(out_dtype), _ptr(out), _stream(stream)))


def svdq_quantize_next_workspace_bytes(cfg, next_cfg, M):
    n = ctypes.c_int64(0)
    _check(lib().svdq_quantize_next_workspace_bytes(ctypes.byref(cfg), ctypes.byref(next_cfg),
                                                    int(M), ctypes.byref(n)))
    return n.value


def svdq_gemm_w4a4_packed_quantize_next(cfg, M, act_packed, prepacked, lora_act, l2, bias, act,
                                        next_cfg, next_smooth_inv, next_l1, next_act_packed,
                                        next_act_scales, next_lora_act, lora_workspace,
                                        stream=None):
    return _check(lib().svdq_gemm_w4a4_packed_quantize_next(
        ctypes.byref(cfg), int(M), _ptr(act_packed), _ptr(prepacked), _ptr(lora_act), _ptr(l2),
        _ptr(bias), int(act), ctypes.byref(next_cfg), _ptr(next_smooth_inv), _ptr(next_l1),
        _ptr(next_act_packed), _ptr(next_act_scales), _ptr(next_lora_act), _ptr(lora_workspace),
        _stream(stream)))


def svdq_calib_absmax(M, K, x, absmax, stream=None):
    return _check(lib().svdq_calib_absmax(int(M), int(K), _ptr(x), _ptr(absmax), _stream(stream)))


def svdq_smoothing_factors(cfg, w, x_absmax, w_absmax, smooth_inv, stream=None):
    return _check(lib().svdq_smoothing_factors(ctypes.byref(cfg), _ptr(w), _ptr(x_absmax),
                                               _ptr(w_absmax), _ptr(smooth_inv), _stream(stream)))


def svdq_quantize_residual(cfg, w, smooth_inv, l1, l2, wgt_codes, wgt_scales, wgt_global_scale=None,
                           stream=None):
    return _check(lib().svdq_quantize_residual(ctypes.byref(cfg), _ptr(w), _ptr(smooth_inv),
                                               _ptr(l1), _ptr(l2), _ptr(wgt_codes), _ptr(wgt_scales),
                                               _ptr(wgt_global_scale), _stream(stream)))


def svdq_lowrank_workspace_bytes(cfg):
    n = ctypes.c_int64(0)
    _check(lib().svdq_lowrank_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)))
    return n.value


def svdq_lowrank_factors(cfg, w, smooth_inv, omega, block, iters, l1, l2, sigma, workspace,
                         stream=None):
    return _check(lib().svdq_lowrank_factors(ctypes.byref(cfg), _ptr(w), _ptr(smooth_inv),
                                             _ptr(omega), int(block), int(iters), _ptr(l1), _ptr(l2),
                                             _ptr(sigma), _ptr(workspace), _stream(stream)))


def svdq_peak_mfma(kind, iters, out, stream=None):
    """Launch the MFMA-rate kernel of `kind`; returns the operations the launch performs."""
    n = ctypes.c_int64(0)
    _check(lib().svdq_peak_mfma(int(kind), int(iters), _ptr(out), ctypes.byref(n), _stream(stream)))
    return n.value


def svdq_peak_copy(src, dst, nbytes, stream=None):
    return _check(lib().svdq_peak_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)))


def svdq_peak_read(src, nbytes, out, stream=None):
    return _check(lib().svdq_peak_read(_ptr(src), int(nbytes), _ptr(out), _stream(stream)))


def svdq_check_device(device=0):
    return lib().svdq_check_device(int(device))


def svdq_check_arch(name):
    return lib().svdq_check_arch(name.encode() if isinstance(name, str) else name)


def svdq_status_string(status):
    return lib().svdq_status_string(int(status)).decode()


def svdq_last_error():
    return lib().svdq_last_error().decode()


def svdq_version():
    return lib().svdq_version()

"""Independent NumPy fp64 formulations used to pin the C oracle.  TEST INFRASTRUCTURE.

These restate the same definitions a different way (exhaustive nearest-code search
instead of divide-and-round; dequantize-then-matmul instead of integer group dots)
so that a slip in one formulation shows up as a disagreement.
"""
import numpy as np

from . import bf16_to_f64, unpack_int4, unpack_u4, e2m1_decode, e4m3_decode


def nearest_int4(xhat_f32, s_f32):
    """For each value, the integer c in [-8, 7] nearest to xhat / s in exact arithmetic,
    ties to even.  Returns (codes, near_tie) where near_tie flags values whose exact
    quotient lies within 2 fp32 ulps of a half-integer (there the fp32 division that
    defines the code may round across the tie)."""
    x = np.asarray(xhat_f32, np.float64)
    s = np.asarray(s_f32, np.float64)
    cands = np.arange(-8, 8, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        t = np.where(s > 0, x / np.where(s > 0, s, 1.0), 0.0)
    # exhaustive: distance |x - c*s| (exact enough in fp64: x, s are fp32)
    d = np.abs(x[..., None] - cands * s[..., None])
    dmin = d.min(axis=-1, keepdims=True)
    is_min = d == dmin
    even = (cands.astype(np.int64) % 2 == 0)
    pick_even = is_min & even
    has_even_tie = pick_even.any(axis=-1)
    idx = np.where(has_even_tie, np.argmax(pick_even, axis=-1), np.argmax(is_min, axis=-1))
    codes = cands[idx].astype(np.int8)
    codes = np.where(s > 0, codes, 0).astype(np.int8)
    frac = np.abs(t - np.floor(t) - 0.5)
    near_tie = (s > 0) & (frac <= 4.0 * np.finfo(np.float32).eps * np.maximum(np.abs(t), 1.0))
    return codes, near_tie


def dequant_int4(codes, scales):
    q = unpack_int4(codes).astype(np.float64)
    R, K = q.shape
    return q * np.repeat(np.asarray(scales, np.float64), 64, axis=1)


def gemm_dequant_int4(ca, sa, cw, sw, lora=None, l2=None, bias=None):
    Y = dequant_int4(ca, sa) @ dequant_int4(cw, sw).T
    if lora is not None and lora.shape[1] > 0:
        Y = Y + bf16_to_f64(lora) @ bf16_to_f64(l2).T
    if bias is not None:
        Y = Y + bf16_to_f64(bias)[None, :]
    return Y


def dequant_nvfp4(codes, scales, S):
    c = unpack_u4(codes)
    vals = e2m1_decode(c.reshape(-1)).reshape(c.shape)
    sb = e4m3_decode(np.asarray(scales).reshape(-1)).reshape(np.asarray(scales).shape)
    return vals * np.repeat(sb, 16, axis=1) * float(S)


def gemm_dequant_nvfp4(ca, sa, Sa, cw, sw, Sw, lora=None, l2=None, bias=None):
    Y = dequant_nvfp4(ca, sa, Sa) @ dequant_nvfp4(cw, sw, Sw).T
    if lora is not None and lora.shape[1] > 0:
        Y = Y + bf16_to_f64(lora) @ bf16_to_f64(l2).T
    if bias is not None:
        Y = Y + bf16_to_f64(bias)[None, :]
    return Y


def dequant_awq(q, sc, z):
    u = unpack_u4(q).astype(np.float64)
    s = np.repeat(bf16_to_f64(sc), 64, axis=1)
    zz = np.repeat(bf16_to_f64(z), 64, axis=1)
    return (u - zz) * s


def lowrank_down_f64(x_bf16, l1_bf16):
    return bf16_to_f64(x_bf16) @ bf16_to_f64(l1_bf16).T

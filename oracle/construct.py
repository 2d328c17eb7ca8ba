"""Offline weight construction (the calibrate-and-quantize step that produces the
tensors both the oracle and the HIP path consume).  TEST INFRASTRUCTURE ONLY.

SVDQuant, as the pages state it (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
Diffusers", 技术细节 1, "SVDQuant 的核心思路"; page "Diffusers Natively Integrates
Nunchaku Lite ...", third paragraph; page "Nunchaku Lite: 4-битная генерация ...",
"Что такое Nunchaku и SVDQuant"):
  1. migrate activation outliers into the weights (per-input-channel smoothing);
  2. carry the hardest part of each smoothed weight in a small 16-bit low-rank branch;
  3. quantize the remaining residual to 4 bits.
Readings used here (the pages give no formula):
  * smoothing factor lambda_j = sqrt(max_m |X[m,j]| / max_n |W[n,j]|), 1 when either max
    is 0 or not finite; smooth_inv = fp32(1 / lambda); lambda_eff = 1 / smooth_inv;
  * the low-rank branch is the top-r singular triplets of W diag(lambda_eff), split as
    sqrt(sigma) on each side; L1 (down, [r, K]) absorbs smooth_inv so the kernel can
    apply it to raw X; L1, L2 are rounded once to bf16;
  * the residual is formed with the *rounded* factors, so X_hat R^T + X L1^T L2^T equals
    X W^T in exact arithmetic; it is rounded to fp32 and quantized by the oracle's
    4-bit rule (INT4 64-groups, or NVFP4 16-blocks under S_w = fp32(max|R| / 2688)).
AWQ (page "Diffusers Natively Integrates ...", third paragraph: modulation layers use
W4A16): per-channel scale s_j = a_j^0.5 from synthetic activation magnitudes a_j;
W' = fp32(W diag(s)), x' = bf16(fp32(x) / s); then the oracle's AWQ quantizer.
"""
import numpy as np

import synth
from . import (awq_quant_weight, bf16_to_f64, quant_rows_int4, quant_rows_nvfp4)


def bf16_from_f64_vec(d):
    """Vectorised nearest-bf16 of binary64 values, one rounding, ties to even."""
    d = np.asarray(d, np.float64)
    a = np.abs(d)
    sign = np.signbit(d)
    with np.errstate(divide="ignore", invalid="ignore"):
        _, e = np.frexp(a)
    q = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(a, -q))
    v = np.ldexp(r, q)
    v = np.where(v > np.ldexp(255.0, 120), np.inf, v)
    f = v.astype(np.float32)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    bits = np.where(sign, bits | 0x8000, bits).astype(np.uint16)
    bits = np.where(np.isnan(d), np.uint16(0x7FC0), bits)
    return bits


def smoothing(x_bf16, w):
    xf = bf16_to_f64(x_bf16)
    cx = np.max(np.abs(xf), axis=0)
    cw = np.max(np.abs(w), axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lam = np.sqrt(cx / cw)
    bad = ~np.isfinite(lam) | (lam == 0) | (cx == 0) | (cw == 0)
    lam = np.where(bad, 1.0, lam)
    smooth_inv = (1.0 / lam).astype(np.float32)
    lam_eff = 1.0 / smooth_inv.astype(np.float64)
    return smooth_inv, lam_eff


def lowrank_residual(w, smooth_inv, lam_eff, rank):
    """Top-r factors of the smoothed weight and the fp64 residual."""
    w_hat = w * lam_eff[None, :]
    if rank > 0:
        U, S, Vt = np.linalg.svd(w_hat, full_matrices=False)
        rs = np.sqrt(S[:rank])
        l1 = bf16_from_f64_vec(rs[:, None] * Vt[:rank, :] * smooth_inv.astype(np.float64)[None, :])
        l2 = bf16_from_f64_vec(U[:, :rank] * rs[None, :])
        R = w_hat - (bf16_to_f64(l2) @ bf16_to_f64(l1)) * lam_eff[None, :]
        sv = S
    else:
        l1 = np.zeros((0, w.shape[1]), np.uint16)
        l2 = np.zeros((w.shape[0], 0), np.uint16)
        R = w_hat.copy()
        sv = None
    return l1, l2, R, sv


def svdq_linear(x_bf16, w, rank, precision="int4", bias_bf16=None, calib_x_bf16=None):
    """Everything one SVDQuant linear consumes.  calib_x_bf16 (default x) sets lambda."""
    calib = x_bf16 if calib_x_bf16 is None else calib_x_bf16
    smooth_inv, lam_eff = smoothing(calib, w)
    l1, l2, R, sv = lowrank_residual(w, smooth_inv, lam_eff, rank)
    R32 = R.astype(np.float32)
    out = dict(smooth_inv=smooth_inv, lam_eff=lam_eff, l1=l1, l2=l2, R=R, R32=R32,
               bias=bias_bf16, rank=rank, precision=precision, singular_values=sv)
    if precision == "int4":
        out["wcodes"], out["wscales"] = quant_rows_int4(R32)
    elif precision == "nvfp4":
        Sw = np.float32(np.max(np.abs(R32)) / np.float32(2688.0))
        out["Sw"] = Sw
        out["wcodes"], out["wscales"] = quant_rows_nvfp4(R32, Sw)
        xhat = synth.bf16_bits_to_f32(x_bf16) * smooth_inv[None, :]
        out["Sa"] = np.float32(np.max(np.abs(xhat)) / np.float32(2688.0))
    else:
        raise ValueError(precision)
    return out


def awq_linear(x_bf16, w, act_magnitude, bias_bf16=None):
    s = np.sqrt(act_magnitude)
    s32 = s.astype(np.float32)
    w_prime = (w * s32.astype(np.float64)[None, :]).astype(np.float32)
    xp = (synth.bf16_bits_to_f32(x_bf16) / s32[None, :]).astype(np.float32)
    x_prime = synth.f32_to_bf16_bits(xp)
    q, sc, z = awq_quant_weight(w_prime)
    return dict(x_prime=x_prime, w_prime=w_prime, qweight=q, scales=sc, zeros=z,
                bias=bias_bf16, s=s32)


def build_workload(wl, M=None, seed_offset=0):
    """Draw a workload and construct its weights.  Returns (draws, layers) where layers is
    a list of dicts (two for the MLP pair)."""
    d = synth.draw(wl, seed_offset=seed_offset, M=M)
    if wl.precision == "awq":
        return d, [awq_linear(d.x_bf16, d.w, d.extras["act_magnitude"], d.bias_bf16)]
    layers = [svdq_linear(d.x_bf16, d.w, wl.rank, wl.precision, d.bias_bf16)]
    if wl.K2:
        layers.append(svdq_linear(d.extras["x2_bf16"], d.extras["w2"], wl.rank, wl.precision,
                                  d.extras["bias2_bf16"]))
    return d, layers

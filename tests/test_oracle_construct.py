"""Pins of the offline weight construction (page "Hugging Face 把 Nunchaku 4-bit Diffusion
接到 Diffusers", 技术细节 1, "SVDQuant 的核心思路" steps 1-3) and a method-level check of
the qualitative claim on the same page that plain W4A4 breaks on outliers while the
SVDQuant combination does not.
"""
import numpy as np

import oracle
import synth
from oracle import bruteforce as bf
from oracle.construct import build_workload, svdq_linear, smoothing


def _tiny():
    return synth.WORKLOADS[0]


def test_smoothing_invariance_with_identity_quantizer():
    # X_hat R^T + X L1^T L2^T == X W^T in exact arithmetic, for any rank.
    d = synth.draw(_tiny(), M=64)
    x = oracle.bf16_to_f64(d.x_bf16)
    for rank in (0, 4, 16):
        L = svdq_linear(d.x_bf16, d.w, rank)
        xhat = x * L["smooth_inv"].astype(np.float64)[None, :]
        lhs = xhat @ L["R"].T
        if rank:
            lhs = lhs + (x @ oracle.bf16_to_f64(L["l1"]).T) @ oracle.bf16_to_f64(L["l2"]).T
        ref = x @ d.w.T
        assert np.max(np.abs(lhs - ref)) <= 1e-10 * np.max(np.abs(ref))


def test_smoothing_factor_definition():
    d = synth.draw(_tiny(), M=64)
    si, lam_eff = smoothing(d.x_bf16, d.w)
    x = oracle.bf16_to_f64(d.x_bf16)
    lam = np.sqrt(np.abs(x).max(0) / np.abs(d.w).max(0))
    assert np.array_equal(si, (1.0 / lam).astype(np.float32))
    assert np.allclose(lam_eff * si, 1.0, rtol=1e-15)
    # outlier channels get the largest factors
    top = np.argsort(lam)[-len(d.outlier_channels):]
    assert set(top) == set(d.outlier_channels.tolist())
    # zero column -> lambda = 1
    xz = d.x_bf16.copy()
    xz[:, 5] = 0
    si2, _ = smoothing(xz, d.w)
    assert si2[5] == 1.0


def test_eckart_young_before_rounding():
    rng = np.random.default_rng(40)
    w = rng.standard_normal((96, 128)) * 0.02
    xb = synth.random_bf16(rng, (32, 128), 1.0)
    r = 8
    L = svdq_linear(xb, w, r)
    w_hat = w * L["lam_eff"][None, :]
    U, S, Vt = np.linalg.svd(w_hat, full_matrices=False)
    approx = (U[:, :r] * S[:r]) @ Vt[:r]
    err = np.linalg.norm(w_hat - approx)
    assert abs(err - np.sqrt(np.sum(S[r:] ** 2))) <= 1e-12 * err
    # the stored (bf16) factors are within bf16 rounding of the exact split
    l2l1 = oracle.bf16_to_f64(L["l2"]) @ oracle.bf16_to_f64(L["l1"]) * L["lam_eff"][None, :]
    assert np.linalg.norm(l2l1 - approx) <= 2 ** -7 * np.linalg.norm(approx)


def _sqnr(ref, y):
    return 10 * np.log10(np.sum(ref ** 2) / np.sum((ref - y) ** 2))


def test_svdquant_beats_naive_w4a4_on_outliers():
    wl = _tiny()
    d, (L,) = build_workload(wl)
    x = oracle.bf16_to_f64(d.x_bf16)
    ref = x @ d.w.T
    ca, sa, lora = oracle.quant_act_int4(d.x_bf16, L["smooth_inv"], L["l1"])
    Y = oracle.gemm_w4a4_int4(ca, sa, L["wcodes"], L["wscales"], lora, L["l2"], None)
    # naive W4A4: no smoothing, no low-rank branch
    ca0, sa0, _ = oracle.quant_act_int4(d.x_bf16, np.ones(wl.K, np.float32))
    cw0, sw0 = oracle.quant_rows_int4(d.w.astype(np.float32))
    Y0 = oracle.gemm_w4a4_int4(ca0, sa0, cw0, sw0)
    s_svdq, s_naive = _sqnr(ref, Y), _sqnr(ref, Y0)
    assert s_svdq > s_naive + 3.0, (s_svdq, s_naive)


def test_workload_shapes_and_seeds():
    wl = _tiny()
    d1, (L1,) = build_workload(wl)
    d2, (L2,) = build_workload(wl)
    assert np.array_equal(d1.x_bf16, d2.x_bf16) and np.array_equal(L1["wcodes"], L2["wcodes"])
    assert d1.x_bf16.shape == (256, 512) and L1["l1"].shape == (16, 512)
    assert L1["l2"].shape == (512, 16) and L1["wcodes"].shape == (512, 256)
    assert len(d1.outlier_channels) == 10 and d1.bias_bf16 is None


def test_dequantized_residual_close_to_residual():
    wl = _tiny()
    _, (L,) = build_workload(wl)
    deq = bf.dequant_int4(L["wcodes"], L["wscales"])
    step = np.repeat(L["wscales"].astype(np.float64), 64, axis=1)
    assert np.all(np.abs(deq - L["R32"]) <= 0.5 * step * (1 + 1e-6) + 1e-30)

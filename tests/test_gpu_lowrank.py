"""GPU top-r factorization of the smoothed weight (randomized subspace iteration) against
the oracle's exact SVD (numpy, binary64).  It approximates the exact factors, so it is
pinned by what the exact SVD fixes: on a weight of rank <= block the triplets are exact (up
to fp32), on a decaying spectrum the leading singular values agree closely, and on a
Gaussian weight of the pages' kind the energy the branch captures (||W_hat||^2 minus the
residual's) is within a stated fraction of what the exact top-r branch captures (Eckart-
Young: no rank-r branch captures more)."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import synth
from oracle import bf16_to_f64
from oracle.construct import lowrank_residual, smoothing

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _factor(w32, si, r, b, iters, rng):
    N, K = w32.shape
    cfg = bd.LayerCfg.make(K, N, r)
    omega = rng.standard_normal((K, b)).astype(np.float32)
    l1 = torch.empty((r, K), dtype=torch.int16, device="cuda:0")
    l2 = torch.empty((N, r), dtype=torch.int16, device="cuda:0")
    sig = torch.empty(r, dtype=torch.float32, device="cuda:0")
    ws = torch.empty(bd.svdq_lowrank_workspace_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    bd.svdq_lowrank_factors(cfg, gu.dev(w32), gu.dev(si), gu.dev(omega), b, iters, l1, l2, sig, ws)
    torch.cuda.synchronize()
    return gu.host(l1).view(np.uint16), gu.host(l2).view(np.uint16), gu.host(sig)


def _captured(w_hat, l1, l2, lam):
    """Energy of W_hat that the branch (bf16 factors, un-smoothed) removes."""
    P = (bf16_to_f64(l2) @ bf16_to_f64(l1)) * lam[None, :]
    return np.sum(w_hat ** 2) - np.sum((w_hat - P) ** 2)


def _case(rng, N, K, kind):
    x = synth.random_bf16(rng, (256, K), 1.0)
    x[:, rng.integers(0, K, 4)] = synth.random_bf16(rng, (256, 4), 30.0)   # outlier channels
    if kind == "rank40":
        w = rng.normal(0, 0.02, (N, 40)) @ rng.normal(0, 1.0, (40, K)) / np.sqrt(40)
    elif kind == "decay":
        U, _ = np.linalg.qr(rng.normal(size=(N, 64)))
        V, _ = np.linalg.qr(rng.normal(size=(K, 64)))
        w = (U * (0.5 * 0.85 ** np.arange(64))) @ V.T + rng.normal(0, 1e-4, (N, K))
    else:
        w = rng.normal(0.0, 0.02, (N, K))
    w32 = w.astype(np.float32)
    w64 = w32.astype(np.float64)
    si, lam = smoothing(x, w64)
    return w32, w64, si, lam


@pytest.mark.parametrize("N,K", [(200, 320), (384, 512)])
def test_lowrank_exact_rank(N, K):
    rng = np.random.default_rng(1700 + N)
    w32, w64, si, lam = _case(rng, N, K, "rank40")
    l1, l2, sig = _factor(w32, si, 32, 48, 1, rng)
    w_hat = w64 * lam[None, :]
    s_ex = np.linalg.svd(w_hat, compute_uv=False)[:32]
    print(f"rank40 sigma rel err {np.max(np.abs(sig - s_ex) / s_ex):.2e}")
    assert np.allclose(sig, s_ex, rtol=1e-4)
    o1, o2, _, _ = lowrank_residual(w64, si, lam, 32)
    P = (bf16_to_f64(l2) @ bf16_to_f64(l1)) * lam[None, :]
    Po = (bf16_to_f64(o2) @ bf16_to_f64(o1)) * lam[None, :]
    e = np.linalg.norm(P - Po) / np.linalg.norm(Po)
    print(f"rank40 branch rel diff {e:.2e}")
    assert e <= 1e-2


@pytest.mark.parametrize("b,r,N,K", [(16, 16, 200, 320), (33, 32, 264, 448), (64, 48, 384, 640)])
def test_lowrank_block_widths_exact_rank(b, r, N, K):
    """Block widths 16, 33 (odd: the eigensolver's round-robin schedule gets a dummy index)
    and 64 (the maximum) on a weight of rank b: the b-column block spans its range, so the
    leading r singular values are the exact SVD's up to fp32."""
    rng = np.random.default_rng(1800 + b)
    x = synth.random_bf16(rng, (256, K), 1.0)
    k = b
    w = rng.normal(0, 0.02, (N, k)) @ rng.normal(0, 1.0, (k, K)) / np.sqrt(k)
    w32 = w.astype(np.float32)
    w64 = w32.astype(np.float64)
    si, lam = smoothing(x, w64)
    _, _, sig = _factor(w32, si, r, b, 1, rng)
    s_ex = np.linalg.svd(w64 * lam[None, :], compute_uv=False)[:r]
    rel = np.max(np.abs(sig - s_ex) / s_ex)
    print(f"b={b} rank {k}: sigma rel err {rel:.2e}")
    assert rel <= 1e-4


def test_lowrank_decaying_spectrum():
    rng = np.random.default_rng(1710)
    w32, w64, si, lam = _case(rng, 384, 512, "decay")
    l1, l2, sig = _factor(w32, si, 32, 48, 3, rng)
    s_ex = np.linalg.svd(w64 * lam[None, :], compute_uv=False)[:32]
    rel = np.abs(sig - s_ex) / s_ex
    print(f"decay sigma rel err first 16 {np.max(rel[:16]):.2e} all {np.max(rel):.2e}")
    assert np.max(rel[:16]) <= 1e-3 and np.max(rel) <= 1e-2


@pytest.mark.parametrize("N,K,r", [(1024, 3072, 32), (3072, 3072, 32)])
def test_lowrank_gaussian_captured_energy(N, K, r):
    rng = np.random.default_rng(1720 + N)
    w32, w64, si, lam = _case(rng, N, K, "gauss")
    l1, l2, _ = _factor(w32, si, r, 48, 4, rng)
    o1, o2, _, _ = lowrank_residual(w64, si, lam, r)
    w_hat = w64 * lam[None, :]
    eg, eo = _captured(w_hat, l1, l2, lam), _captured(w_hat, o1, o2, lam)
    print(f"gauss {N}x{K} captured energy ratio {eg / eo:.4f}")
    assert eg <= eo * (1 + 1e-3) and eg >= 0.95 * eo


def test_lowrank_attention_weight_captured_energy():
    # the attention projection's own smoothed weight (3072 x 3072, calibration from its
    # 4096-token draw with 31 outlier channels x50) at the benchmark's settings (block 48,
    # four iterations): its 31 outlier directions stand well above the bulk, so the branch
    # captures all but a sliver of what the exact top-32 branch does
    wl = synth.WORKLOADS[1]
    d = synth.draw(wl)
    w64 = d.w.astype(np.float32).astype(np.float64)
    si, lam = smoothing(d.x_bf16, w64)
    rng = np.random.default_rng(1730)
    l1, l2, sig = _factor(w64.astype(np.float32), si, 32, 48, 4, rng)
    o1, o2, _, _ = lowrank_residual(w64, si, lam, 32)
    w_hat = w64 * lam[None, :]
    eg, eo = _captured(w_hat, l1, l2, lam), _captured(w_hat, o1, o2, lam)
    print(f"attention weight captured energy ratio {eg / eo:.6f}")
    assert eg <= eo * (1 + 1e-4) and eg >= 0.999 * eo

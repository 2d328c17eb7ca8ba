"""GPU parity of the offline weight quantizer against the oracle's construction, bit for
bit: the calibration absmax (accumulated over two batches), the smoothing factors (including
channels whose activation or weight maximum is zero), and the INT4 residual's codes and
scales given the oracle's top-r factors, INT4 and NVFP4 (with its per-tensor scale), at
ranks 0 to 64 and on a 3072-channel layer."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import oracle
import synth
from oracle.construct import lowrank_residual, smoothing

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _calib(x_list, K):
    am = torch.zeros(K, dtype=torch.float32, device="cuda:0")
    for x in x_list:
        bd.svdq_calib_absmax(x.shape[0], K, gu.dev(x), am)
    return am


@pytest.mark.parametrize("M,K", [(1, 64), (300, 320), (4096, 3072)])
def test_calib_absmax(M, K):
    rng = np.random.default_rng(1600 + M + K)
    x1 = synth.random_bf16(rng, (M, K), 1.0)
    x2 = synth.random_bf16(rng, (M // 2 + 1, K), 1.0)
    x2[:, 7] = synth.random_bf16(rng, (x2.shape[0], 1), 40.0)[:, 0]   # an outlier channel
    am = gu.host(_calib([x1, x2], K))
    ref = np.max(np.abs(synth.bf16_bits_to_f32(np.concatenate([x1, x2]))), axis=0)
    assert np.array_equal(am.view(np.uint32), ref.astype(np.float32).view(np.uint32))


@pytest.mark.parametrize("N,K", [(200, 320), (3072, 3072)])
def test_smoothing_factors(N, K):
    rng = np.random.default_rng(1610 + N + K)
    x = synth.random_bf16(rng, (257, K), 1.0)
    x[:, 3] = 0                                         # activation maximum 0 -> lambda 1
    x[:, 11] = synth.random_bf16(rng, (257, 1), 60.0)[:, 0]
    w = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    w[:, 5] = 0.0                                       # weight maximum 0 -> lambda 1
    cfg = bd.LayerCfg.make(K, N, 0)
    am = _calib([x], K)
    wam = torch.empty(K, dtype=torch.float32, device="cuda:0")
    si = torch.empty(K, dtype=torch.float32, device="cuda:0")
    bd.svdq_smoothing_factors(cfg, gu.dev(w), am, wam, si)
    osi, _ = smoothing(x, w.astype(np.float64))
    assert np.array_equal(gu.host(wam), np.max(np.abs(w), axis=0))
    assert np.array_equal(gu.host(si).view(np.uint32), osi.view(np.uint32))
    assert gu.host(si)[3] == 1.0 and gu.host(si)[5] == 1.0


@pytest.mark.parametrize("N,K,r", [(200, 320, 16), (384, 512, 32), (96, 128, 0), (130, 256, 64),
                                   (1024, 3072, 32)])
def test_quantize_residual(N, K, r):
    """Given the oracle's smoothing factors and top-r factors, the residual's codes and scales
    equal the oracle's quantization of its fp64 residual rounded to fp32."""
    rng = np.random.default_rng(1620 + N + K + r)
    print(f"residual N={N} K={K} r={r}", flush=True)
    x = synth.random_bf16(rng, (128, K), 1.0)
    cols = rng.integers(0, K, 4)
    x[:, cols] = synth.random_bf16(rng, (128, 4), 30.0)   # outlier channels
    w = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    w64 = w.astype(np.float64)
    si, lam = smoothing(x, w64)
    l1, l2, R, _ = lowrank_residual(w64, si, lam, r)
    oc, os_ = oracle.quant_rows_int4(R.astype(np.float32))
    cfg = bd.LayerCfg.make(K, N, r)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((N, K // 64), dtype=torch.float32, device="cuda:0")
    bd.svdq_quantize_residual(cfg, gu.dev(w), gu.dev(si), gu.dev(l1) if r else None,
                              gu.dev(l2) if r else None, codes, scales)
    gc, gs = gu.host(codes), gu.host(scales)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"
    assert np.array_equal(gc, oc), f"codes differ in {np.count_nonzero(gc != oc)} bytes"


@pytest.mark.parametrize("N,K,r", [(200, 320, 16), (96, 128, 0), (1024, 3072, 32)])
def test_quantize_residual_nvfp4(N, K, r):
    """NVFP4: S_w = fp32(max |R32| / 2688), then E4M3 block scales and E2M1 codes, against
    the oracle's construction bit for bit."""
    rng = np.random.default_rng(1640 + N + K + r)
    print(f"residual nvfp4 N={N} K={K} r={r}", flush=True)
    x = synth.random_bf16(rng, (128, K), 1.0)
    w = rng.normal(0.0, 0.02, (N, K)).astype(np.float32)
    w[3, 17] = 0.9                                     # one large weight sets S_w
    w64 = w.astype(np.float64)
    si, lam = smoothing(x, w64)
    l1, l2, R, _ = lowrank_residual(w64, si, lam, r)
    R32 = R.astype(np.float32)
    Sw = np.float32(np.max(np.abs(R32)) / np.float32(2688.0))
    oc, os_ = oracle.quant_rows_nvfp4(R32, Sw)
    cfg = bd.LayerCfg.make(K, N, r, "nvfp4")
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda:0")
    gs = torch.empty(1, dtype=torch.float32, device="cuda:0")
    bd.svdq_quantize_residual(cfg, gu.dev(w), gu.dev(si), gu.dev(l1) if r else None,
                              gu.dev(l2) if r else None, codes, scales, gs)
    assert gu.host(gs).view(np.uint32)[0] == np.array([Sw], np.float32).view(np.uint32)[0]
    assert np.array_equal(gu.host(scales), os_), "block scales differ"
    gc = gu.host(codes)
    assert np.array_equal(gc, oc), f"codes differ in {np.count_nonzero(gc != oc)} bytes"

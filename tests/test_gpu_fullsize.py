"""GPU parity at the full workload sizes, in the launch configuration the benchmark times:
  attention projection 4096x3072x3072 r32 (INT4), the DiT MLP pair 4608x3072->12288->3072
  with GELU (INT4), the fused-QKV NVFP4 projection 4096x3072x9216 r32, the AWQ GEMV
  2x3072x18432, the MLP with fc2's activation kernel fused into fc1's epilogue, and the
  offline weight quantizer.  Weights come from the oracle's offline construction
  (smoothing factors, top-r factors, quantized residual).

Per stage, the GPU kernel is fed the oracle's inputs (never the other way round): the
activation kernel is compared in full (codes and scales bit-exact, lora_act within its
bound); the GEMM, fed the oracle's activation-stage outputs, on sampled elements (random
points, whole rows and whole columns) that the oracle computes one by one.  End to end,
the GPU chain and the oracle chain each run from the same X and are compared.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.construct import bf16_from_f64_vec, build_workload

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

gu = pytest.importorskip("gpu_util")


def _get(cache, idx):
    if idx not in cache:
        cache[idx] = build_workload(synth.WORKLOADS[idx])
    return cache[idx]


def _samples(rng, M, N, n_pts=3000):
    mi = rng.integers(0, M, n_pts)
    ni = rng.integers(0, N, n_pts)
    rows = np.array([0, M - 1, M // 2])
    cols = np.array([0, N - 1])
    mi = np.concatenate([mi, np.repeat(rows, N), np.tile(np.arange(M), len(cols))])
    ni = np.concatenate([ni, np.tile(np.arange(N), len(rows)), np.repeat(cols, M)])
    return mi, ni


def _quant_exact(xb, L, precision="int4", S=1.0):
    """GPU activation kernel vs oracle on the same input; returns both."""
    codes, scales, lora = gu.quantize(xb, L["smooth_inv"], L["l1"], precision, float(S))
    torch.cuda.synchronize()
    if precision == "int4":
        oc, os_, ol = oracle.quant_act_int4(xb, L["smooth_inv"], L["l1"])
    else:
        oc, os_, ol = oracle.quant_act_nvfp4(xb, L["smooth_inv"], S, L["l1"])
    gc, gs, gl = gu.host(codes), gu.host(scales), gu.host(lora)
    assert np.array_equal(gc, oc), f"codes differ in {np.count_nonzero(gc != oc)} bytes"
    assert np.array_equal(gs.view(np.uint8), os_.view(np.uint8)), "scales differ"
    gu.assert_lora_close(gl, ol, xb, L["l1"])
    return (codes, scales, lora), (oc, os_, ol)


def test_attn_projection_int4(workload_cache):
    d, (L,) = _get(workload_cache, 1)
    (gc, gs, gl), (oc, os_, ol) = _quant_exact(d.x_bf16, L)
    rng = np.random.default_rng(1)
    # GEMM stage on the oracle's activation-stage outputs
    y = gu.host(gu.gemm(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"]))
    mi, ni = _samples(rng, *y.shape)
    ref = oracle.gemm_w4a4_int4_at(mi, ni, oc, os_, L["wcodes"], L["wscales"], ol, L["l2"],
                                   L["bias"])
    e = gu.rel_fro(y[mi, ni], ref)
    print(f"attn int4 gemm rel_fro={e:.3e}")
    assert e <= 1e-3
    K = d.x_bf16.shape[1]
    cond = gu.int4_cond(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"], mi, ni)
    gu.assert_f32_within(y[mi, ni], ref, cond, gu.int4_nround(K, L["rank"]))
    yb = gu.host(gu.gemm(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"],
                         out_bf16=True))
    gu.assert_bf16_close(yb[mi, ni], ref, cond, gu.int4_nround(K, L["rank"]))
    # end to end: GPU chain vs oracle chain from the same X
    ye = gu.host(gu.gemm(gc, gs, L["wcodes"], L["wscales"], gl, L["l2"], L["bias"]))
    e2e = gu.rel_fro(ye[mi, ni], ref)
    print(f"attn int4 end-to-end rel_fro={e2e:.3e}")
    assert e2e <= 1e-3


def test_mlp_pair_int4(workload_cache):
    d, (L1, L2) = _get(workload_cache, 2)
    rng = np.random.default_rng(2)
    # fc1: activation kernel in full, then GEMM with fused GELU and bf16 output
    (gc1, gs1, gl1), (oc1, os1, ol1) = _quant_exact(d.x_bf16, L1)
    h_or = gu.host(gu.gemm(oc1, os1, L1["wcodes"], L1["wscales"], ol1, L1["l2"], L1["bias"],
                           act=1, out_bf16=True))
    mi1, ni1 = _samples(rng, *h_or.shape, n_pts=2000)
    ref1 = oracle.gemm_w4a4_int4_at(mi1, ni1, oc1, os1, L1["wcodes"], L1["wscales"], ol1,
                                    L1["l2"], L1["bias"], act=1)
    # bf16 rounding alone is ~1.5e-3 relative: compare at the same rounding point
    cond1 = gu.int4_cond(oc1, os1, L1["wcodes"], L1["wscales"], ol1, L1["l2"], L1["bias"], mi1, ni1)
    gu.assert_bf16_close(h_or[mi1, ni1], ref1, cond1, gu.int4_nround(d.x_bf16.shape[1], L1["rank"]),
                         gelu=True)
    # the oracle's chain on a few token rows: fc1 -> GELU (fp64) -> bf16 -> fc2
    rows = np.array([0, 1, 777, 2048, 4095, d.x_bf16.shape[0] - 1])
    y1 = oracle.gemm_w4a4_int4(oc1[rows], os1[rows], L1["wcodes"], L1["wscales"], ol1[rows],
                               L1["l2"], L1["bias"], act=1)
    h_rows = bf16_from_f64_vec(y1)
    # fc2's activation kernel on the oracle's intermediate rows: bit-exact
    _, (qc, qs, ql) = _quant_exact(h_rows, L2)
    y2 = oracle.gemm_w4a4_int4(qc, qs, L2["wcodes"], L2["wscales"], ql, L2["l2"], L2["bias"])
    # GPU chain end to end: quant -> GEMM+GELU (bf16) -> quant -> GEMM
    h = gu.gemm(gc1, gs1, L1["wcodes"], L1["wscales"], gl1, L1["l2"], L1["bias"], act=1,
                out_bf16=True)
    c2, s2, lo2 = gu.quantize(h, L2["smooth_inv"], L2["l1"])
    y = gu.host(gu.gemm(c2, s2, L2["wcodes"], L2["wscales"], lo2, L2["l2"], L2["bias"]))
    e2e = gu.rel_fro(y[rows], y2)
    print(f"mlp end-to-end rel_fro={e2e:.3e}")
    assert e2e <= 1e-3
    # fc2 standalone on its heavy-tailed calibration input
    _, (oc3, os3, ol3) = _quant_exact(d.extras["x2_bf16"], L2)
    y3 = gu.host(gu.gemm(oc3, os3, L2["wcodes"], L2["wscales"], ol3, L2["l2"], L2["bias"]))
    mi3, ni3 = _samples(rng, *y3.shape, n_pts=2000)
    ref3 = oracle.gemm_w4a4_int4_at(mi3, ni3, oc3, os3, L2["wcodes"], L2["wscales"], ol3,
                                    L2["l2"], L2["bias"])
    e3 = gu.rel_fro(y3[mi3, ni3], ref3)
    print(f"mlp fc2 gemm rel_fro={e3:.3e}")
    assert e3 <= 1e-3
    cond3 = gu.int4_cond(oc3, os3, L2["wcodes"], L2["wscales"], ol3, L2["l2"], L2["bias"], mi3, ni3)
    gu.assert_f32_within(y3[mi3, ni3], ref3, cond3, gu.int4_nround(L2["wcodes"].shape[1] * 2, L2["rank"]))


def test_qkv_nvfp4(workload_cache):
    d, (L,) = _get(workload_cache, 3)
    (gc, gs, gl), (oc, os_, ol) = _quant_exact(d.x_bf16, L, "nvfp4", L["Sa"])
    kw = dict(precision="nvfp4", Sa=float(L["Sa"]), Sw=float(L["Sw"]))
    y = gu.host(gu.gemm(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"], **kw))
    rng = np.random.default_rng(3)
    mi, ni = _samples(rng, *y.shape)
    ref = oracle.gemm_w4a4_nvfp4_at(mi, ni, oc, os_, L["Sa"], L["wcodes"], L["wscales"],
                                    L["Sw"], ol, L["l2"], L["bias"])
    e = gu.rel_fro(y[mi, ni], ref)
    print(f"qkv nvfp4 gemm rel_fro={e:.3e}")
    assert e <= 1e-3
    cond = gu.nvfp4_cond(oc, os_, L["Sa"], L["wcodes"], L["wscales"], L["Sw"], ol, L["l2"],
                         L["bias"], mi, ni)
    nr = gu.nvfp4_nround(d.x_bf16.shape[1], L["rank"])
    gu.assert_f32_within(y[mi, ni], ref, cond, nr)
    yb = gu.host(gu.gemm(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"],
                         out_bf16=True, **kw))
    gu.assert_bf16_close(yb[mi, ni], ref, cond, nr)
    ye = gu.host(gu.gemm(gc, gs, L["wcodes"], L["wscales"], gl, L["l2"], L["bias"], **kw))
    assert gu.rel_fro(ye[mi, ni], ref) <= 1e-3


def test_awq_modulation_gemv(workload_cache):
    d, (A,) = _get(workload_cache, 4)
    y = gu.host(gu.awq(A["x_prime"], A["qweight"], A["scales"], A["zeros"], A["bias"]))
    ref = oracle.awq_gemv(A["x_prime"], A["qweight"], A["scales"], A["zeros"], A["bias"])
    e = gu.rel_fro(y, ref)
    print(f"awq rel_fro={e:.3e}")
    assert e <= 1e-3
    cond = gu.awq_cond(A["x_prime"], A["qweight"], A["scales"], A["zeros"], A["bias"])
    nr = gu.awq_nround(A["x_prime"].shape[1])
    gu.assert_f32_within(y, ref, cond, nr)
    yb = gu.host(gu.awq(A["x_prime"], A["qweight"], A["scales"], A["zeros"], A["bias"],
                        out_bf16=True))
    gu.assert_bf16_close(yb, ref, cond, nr, min_exact=gu.AWQ_MIN_EXACT)


def _quant_packed_exact(xb, L):
    """GPU fused quantize-and-pack vs oracle on the same input: codes read back from the
    packed buffer and fp32 scales bit-exact, lora_act within its bound."""
    M, K = xb.shape
    buf, scales, lora = gu.quantize_packed(xb, L["smooth_inv"], L["l1"])
    torch.cuda.synchronize()
    oc, os_, ol = oracle.quant_act_int4(xb, L["smooth_inv"], L["l1"])
    q, words, canonical = gu.decode_act_packed(gu.host(buf), M, K)
    assert canonical
    assert np.array_equal(q[:M], oracle.unpack_int4(oc).astype(np.int64)), "codes differ"
    assert np.array_equal(gu.host(scales).view(np.uint32), os_.view(np.uint32)), "scales differ"
    assert np.array_equal(words[:M], gu.split_words(os_)), "scale words differ"
    gu.assert_lora_close(gu.host(lora), ol, xb, L["l1"])
    return (buf, lora), (oc, os_, ol)


def test_attn_projection_packed(workload_cache):
    """The benchmark's path: svdq_quantize_act_packed + svdq_gemm_w4a4_packed."""
    d, (L,) = _get(workload_cache, 1)
    M, K = d.x_bf16.shape
    N = L["wcodes"].shape[0]
    (buf, gl), (oc, os_, ol) = _quant_packed_exact(d.x_bf16, L)
    wp = gu.prepack(L["wcodes"], L["wscales"], K, N)
    rng = np.random.default_rng(11)
    # GEMM stage on the oracle's activation-stage outputs
    ap = gu.pack_act(oc, os_, K)
    mi, ni = _samples(rng, M, N)
    ref = oracle.gemm_w4a4_int4_at(mi, ni, oc, os_, L["wcodes"], L["wscales"], ol, L["l2"],
                                   L["bias"])
    cond = gu.int4_cond(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], L["bias"], mi, ni)
    nr = gu.int4_nround(K, L["rank"])
    for out_bf16 in (False, True):
        y = gu.host(gu.gemm_packed(ap, wp, M, K, N, ol, L["l2"], L["bias"], out_bf16=out_bf16))
        if out_bf16:
            gu.assert_bf16_close(y[mi, ni], ref, cond, nr)
        else:
            e = gu.rel_fro(y[mi, ni], ref)
            print(f"attn packed gemm rel_fro={e:.3e}")
            assert e <= 1e-3
            gu.assert_f32_within(y[mi, ni], ref, cond, nr)
    # end to end: GPU chain vs oracle chain from the same X (fp32 output: bf16 rounding
    # alone is ~1e-3 relative and is checked element-wise above)
    ye = gu.host(gu.gemm_packed(buf, wp, M, K, N, gl, L["l2"], L["bias"]))
    ref = oracle.gemm_w4a4_int4_at(mi, ni, oc, os_, L["wcodes"], L["wscales"], ol, L["l2"],
                                   L["bias"])
    e2e = gu.rel_fro(ye[mi, ni], ref)
    print(f"attn packed end-to-end rel_fro={e2e:.3e}")
    assert e2e <= 1e-3


def test_mlp_pair_packed(workload_cache):
    """fc1 (GELU, bf16 out) and fc2 (K = 12288) on the packed path."""
    d, (L1, L2) = _get(workload_cache, 2)
    M, K1 = d.x_bf16.shape
    N1 = L1["wcodes"].shape[0]
    N2 = L2["wcodes"].shape[0]
    rng = np.random.default_rng(12)
    (b1, gl1), (oc1, os1, ol1) = _quant_packed_exact(d.x_bf16, L1)
    wp1 = gu.prepack(L1["wcodes"], L1["wscales"], K1, N1)
    h_or = gu.host(gu.gemm_packed(gu.pack_act(oc1, os1, K1), wp1, M, K1, N1, ol1, L1["l2"],
                                  L1["bias"], act=1, out_bf16=True))
    mi1, ni1 = _samples(rng, M, N1, n_pts=2000)
    ref1 = oracle.gemm_w4a4_int4_at(mi1, ni1, oc1, os1, L1["wcodes"], L1["wscales"], ol1,
                                    L1["l2"], L1["bias"], act=1)
    cond1 = gu.int4_cond(oc1, os1, L1["wcodes"], L1["wscales"], ol1, L1["l2"], L1["bias"], mi1, ni1)
    gu.assert_bf16_close(h_or[mi1, ni1], ref1, cond1, gu.int4_nround(K1, L1["rank"]), gelu=True)
    # fc2 on its heavy-tailed calibration input: quantize-and-pack exact, GEMM sampled (fp32
    # output with the workspace: the launch configuration the benchmark times, K split)
    x2 = d.extras["x2_bf16"]
    _, (oc3, os3, ol3) = _quant_packed_exact(x2, L2)
    wp2 = gu.prepack(L2["wcodes"], L2["wscales"], L2["wcodes"].shape[1] * 2, N2)
    assert gu.split_workspace_bytes(x2.shape[0], x2.shape[1], N2) > 0
    y3 = gu.host(gu.gemm_packed(gu.pack_act(oc3, os3, x2.shape[1]), wp2, x2.shape[0],
                                x2.shape[1], N2, ol3, L2["l2"], L2["bias"], split=True))
    mi3, ni3 = _samples(rng, *y3.shape, n_pts=2000)
    ref3 = oracle.gemm_w4a4_int4_at(mi3, ni3, oc3, os3, L2["wcodes"], L2["wscales"], ol3,
                                    L2["l2"], L2["bias"])
    e3 = gu.rel_fro(y3[mi3, ni3], ref3)
    print(f"mlp fc2 packed gemm rel_fro={e3:.3e}")
    assert e3 <= 1e-3
    cond3 = gu.int4_cond(oc3, os3, L2["wcodes"], L2["wscales"], ol3, L2["l2"], L2["bias"], mi3, ni3)
    gu.assert_f32_within(y3[mi3, ni3], ref3, cond3, gu.int4_nround(x2.shape[1], L2["rank"]))
    # GPU chain end to end on a few token rows against the oracle chain
    h = gu.gemm_packed(b1, wp1, M, K1, N1, gl1, L1["l2"], L1["bias"], act=1, out_bf16=True)
    b2, _, lo2 = gu.quantize_packed(h, L2["smooth_inv"], L2["l1"])
    y = gu.host(gu.gemm_packed(b2, wp2, M, N1, N2, lo2, L2["l2"], L2["bias"], split=True))
    rows = np.array([0, 1, 777, 2048, 4095, M - 1])
    y1 = oracle.gemm_w4a4_int4(oc1[rows], os1[rows], L1["wcodes"], L1["wscales"], ol1[rows],
                               L1["l2"], L1["bias"], act=1)
    qc, qs, ql = oracle.quant_act_int4(bf16_from_f64_vec(y1), L2["smooth_inv"], L2["l1"])
    y2 = oracle.gemm_w4a4_int4(qc, qs, L2["wcodes"], L2["wscales"], ql, L2["l2"], L2["bias"])
    e2e = gu.rel_fro(y[rows], y2)
    print(f"mlp packed end-to-end rel_fro={e2e:.3e}")
    assert e2e <= 1e-3


def test_mlp_fused_epilogue_fullsize(workload_cache):
    """The MLP pair with fc2's activation kernel fused into fc1's epilogue, at the full size
    and in the launch configuration the benchmark times: fc2's packed codes, scale words and
    fp32 scales bit-identical to fc1 (bf16 out) followed by fc2's activation kernel, and
    fc2's lora_act on sampled rows within the fp32 bound of the oracle's down-projection of
    the same bf16 intermediate."""
    d, (L1, L2) = _get(workload_cache, 2)
    M, K1 = d.x_bf16.shape
    N1 = L1["wcodes"].shape[0]
    b1, _, gl1 = gu.quantize_packed(d.x_bf16, L1["smooth_inv"], L1["l1"])
    wp1 = gu.prepack(L1["wcodes"], L1["wscales"], K1, N1)
    h = gu.gemm_packed(b1, wp1, M, K1, N1, gl1, L1["l2"], L1["bias"], act=1, out_bf16=True)
    ub, us, _ = gu.quantize_packed(h, L2["smooth_inv"], L2["l1"])
    fb, fs, fl = gu.gemm_packed_quantize_next(b1, wp1, M, K1, N1, gl1, L1["l2"], L1["bias"], 1,
                                              L2["smooth_inv"], L2["l1"])
    torch.cuda.synchronize()
    assert torch.equal(fb, ub), f"packed bytes differ in {int((fb != ub).sum())} places"
    assert torch.equal(fs.view(torch.int32), us.view(torch.int32)), "fp32 scales differ"
    rng = np.random.default_rng(22)
    rows = np.unique(np.concatenate([rng.integers(0, M, 60), [0, M - 1]]))
    hb = gu.host(h)[rows]
    ol = oracle.quant_act_int4(hb, L2["smooth_inv"], L2["l1"])[2]
    gu.assert_lora_close(gu.host(fl)[rows], ol, hb, L2["l1"])


def test_weight_quantizer_fullsize(workload_cache):
    """The offline weight quantizer on the attention projection's weight (3072 x 3072, rank
    32, 4096 calibration tokens), bit-exact against the oracle's construction from the same
    fp32 weight: calibration absmax, smoothing factors, INT4 residual codes and scales."""
    import bit_diffusion_amd as bd
    from oracle.construct import lowrank_residual, smoothing
    d, (L,) = _get(workload_cache, 1)
    w32 = np.ascontiguousarray(d.w.astype(np.float32))
    N, K = w32.shape
    r = L["rank"]
    cfg = bd.LayerCfg.make(K, N, r)
    am = torch.zeros(K, dtype=torch.float32, device="cuda:0")
    bd.svdq_calib_absmax(d.x_bf16.shape[0], K, gu.dev(d.x_bf16), am)
    wam = torch.empty(K, dtype=torch.float32, device="cuda:0")
    si = torch.empty(K, dtype=torch.float32, device="cuda:0")
    wd = gu.dev(w32)
    bd.svdq_smoothing_factors(cfg, wd, am, wam, si)
    osi, lam = smoothing(d.x_bf16, w32.astype(np.float64))
    assert np.array_equal(gu.host(si).view(np.uint32), osi.view(np.uint32))
    l1, l2, R, _ = lowrank_residual(w32.astype(np.float64), osi, lam, r)
    oc, os_ = oracle.quant_rows_int4(R.astype(np.float32))
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((N, K // 64), dtype=torch.float32, device="cuda:0")
    bd.svdq_quantize_residual(cfg, wd, si, gu.dev(l1), gu.dev(l2), codes, scales)
    assert np.array_equal(gu.host(scales).view(np.uint32), os_.view(np.uint32)), "scales differ"
    gc = gu.host(codes)
    assert np.array_equal(gc, oc), f"codes differ in {np.count_nonzero(gc != oc)} bytes"

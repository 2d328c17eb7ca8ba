"""GPU parity of the INT4 path (activation kernel + W4A4 GEMM) against the CPU oracle, through
the C ABI, on small shapes that span several tiles and ragged tails.

Bar: codes and scales bit-exact; lora_act within 1 bf16 ulp plus the fp32 summation error
bound (>= 99% equal to the oracle); GEMM outputs
within relative Frobenius error 1e-3 of the oracle's fp64 result (fp32 output); bf16 output
within one bf16 ulp of the oracle (plus 2^-16 of the output's largest magnitude for elements
that cancel to near zero), >= 99% of elements equal to the oracle rounded to bf16.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.construct import build_workload, bf16_from_f64_vec

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def _x(rng, M, K, outliers=3, scale=40.0):
    x = rng.standard_normal((M, K)).astype(np.float32)
    if outliers:
        ch = rng.choice(K, outliers, replace=False)
        x[:, ch] *= scale
    return synth.f32_to_bf16_bits(x)


def _check_quant(xb, si, l1, tag=""):
    codes, scales, lora = gu.quantize(xb, si, l1)
    torch.cuda.synchronize()
    oc, os_, ol = oracle.quant_act_int4(xb, si, l1)
    gc, gs = gu.host(codes), gu.host(scales)
    assert np.array_equal(gc, oc), f"{tag}: codes differ at {np.argwhere(gc != oc)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"{tag}: scales differ"
    if l1 is not None and l1.shape[0]:
        gu.assert_lora_close(gu.host(lora), ol, xb, l1)
    return codes, scales, lora


@pytest.mark.parametrize("M,K,r", [(1, 64, 0), (3, 192, 16), (17, 512, 16), (64, 512, 32),
                                   (255, 1024, 48), (300, 320, 128)])
def test_quant_int4_shapes(M, K, r):
    rng = np.random.default_rng(100 + M + K + r)
    xb = _x(rng, M, K)
    si = rng.uniform(0.02, 2.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05) if r else None
    _check_quant(xb, si, l1, f"M{M}K{K}r{r}")


def test_quant_int4_edge_values():
    rng = np.random.default_rng(101)
    M, K = 40, 256
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[0, :64] = 0.0                          # zero group
    x[1, 64:128] = -0.0
    x[2, :] *= 1e-38                         # subnormal range scales
    x[3, :] *= 3e37                          # near the top of the range
    x[4, 5] = 1e4                            # single huge outlier in a group
    vals = np.array([3.5, -3.5, 1.25, -1.25, 0.75, 0.25, -0.25, 1.75, -1.75, 2.25, 2.75,
                     -0.75, 0.5, 3.0, 0.0], np.float32)
    x[5, :] = 0.0
    x[5, :15] = vals                          # exact ties (hand-worked fixture)
    # rows of exact ties: multiples of s/2 with absmax 7 s, s = 2^e
    for i in range(6, 20):
        e = float(2.0 ** rng.integers(-10, 10))
        c = rng.integers(-14, 15, size=K) / 2.0
        c[::64] = 7.0
        x[i] = (c * e).astype(np.float32)
    xb = synth.f32_to_bf16_bits(x)
    for si in (np.ones(K, np.float32), rng.uniform(0.5, 2.0, K).astype(np.float32)):
        _check_quant(xb, si, None, "edge")
    codes, _, _ = gu.quantize(xb, np.ones(K, np.float32))
    q = oracle.unpack_int4(gu.host(codes))
    assert np.array_equal(q[5, :15], [7, -7, 2, -2, 2, 0, 0, 4, -4, 4, 6, -2, 1, 6, 0])


def _rand_gemm_inputs(rng, M, N, K, r, bias=True):
    ca, cw = synth.random_packed_nibbles(rng, M, K), synth.random_packed_nibbles(rng, N, K)
    sa = rng.uniform(0.01, 1.0, (M, K // 64)).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    lora = synth.random_bf16(rng, (M, r), 1.0) if r else None
    l2 = synth.random_bf16(rng, (N, r), 0.1) if r else None
    b = synth.random_bf16(rng, (N,), 0.3) if bias else None
    return ca, sa, cw, sw, lora, l2, b


@pytest.mark.parametrize("M,N,K,r,bias,act", [
    (1, 128, 64, 0, False, 0), (5, 96, 192, 16, True, 0), (130, 200, 512, 32, True, 0),
    (257, 384, 256, 16, True, 1), (64, 128, 1024, 128, False, 1), (33, 17, 128, 0, True, 0),
])
def test_gemm_int4_shapes(M, N, K, r, bias, act):
    rng = np.random.default_rng(200 + M + N + K + r)
    ca, sa, cw, sw, lora, l2, b = _rand_gemm_inputs(rng, M, N, K, r, bias)
    ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw, lora, l2, b, act)
    y = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b, act))
    e = gu.rel_fro(y, ref)
    assert e <= 1e-3, e
    assert e <= 1e-5, f"fp32 output unexpectedly far from the oracle: {e}"
    cond = gu.int4_cond(ca, sa, cw, sw, lora, l2, b)
    gu.assert_f32_within(y, ref, cond, gu.int4_nround(K, r), gelu=act == 1)
    yb = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b, act, out_bf16=True))
    gu.assert_bf16_close(yb, ref, cond, gu.int4_nround(K, r), gelu=act == 1)


def test_gemm_int4_extreme_codes():
    # every code -8 or 7 (largest products), and codes of -8 in the weights only
    M, N, K = 70, 130, 256
    ca = np.full((M, K // 2), 0x77, np.uint8)
    cw = np.full((N, K // 2), 0x88, np.uint8)
    sa = np.full((M, K // 64), 0.5, np.float32)
    sw = np.full((N, K // 64), 0.25, np.float32)
    ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw)
    y = gu.host(gu.gemm(ca, sa, cw, sw))
    assert np.array_equal(y, ref.astype(np.float32))


def test_tiny_workload_end_to_end():
    wl = synth.WORKLOADS[0]
    d, (L,) = build_workload(wl)
    codes, scales, lora = _check_quant(d.x_bf16, L["smooth_inv"], L["l1"], "tiny")
    y = gu.host(gu.gemm(codes, scales, L["wcodes"], L["wscales"], lora, L["l2"], None))
    oc, os_, ol = oracle.quant_act_int4(d.x_bf16, L["smooth_inv"], L["l1"])
    ref = oracle.gemm_w4a4_int4(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], None)
    assert gu.rel_fro(y, ref) <= 1e-3
    # and the method did its job: close to the unquantized product
    exact = oracle.bf16_to_f64(d.x_bf16) @ d.w.T
    assert gu.rel_fro(y, exact) < 0.2


def test_determinism():
    rng = np.random.default_rng(300)
    M, N, K, r = 200, 256, 512, 32
    xb = _x(rng, M, K)
    si = rng.uniform(0.1, 1.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05)
    a1 = [gu.host(t) for t in gu.quantize(xb, si, l1)]
    a2 = [gu.host(t) for t in gu.quantize(xb, si, l1)]
    for u, v in zip(a1, a2):
        assert np.array_equal(u, v)
    ca, sa, cw, sw, lora, l2, b = _rand_gemm_inputs(rng, M, N, K, r)
    y1 = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b))
    y2 = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b))
    assert np.array_equal(y1, y2)


def test_empty_batch_is_a_no_op():
    import bit_diffusion_amd as bd
    cfg = bd.LayerCfg.make(128, 64, 16)
    x = torch.empty((0, 128), dtype=torch.int16, device="cuda:0")
    si = torch.ones(128, dtype=torch.float32, device="cuda:0")
    l1 = torch.zeros((16, 128), dtype=torch.int16, device="cuda:0")
    c = torch.empty((1, 64), dtype=torch.uint8, device="cuda:0")
    s = torch.empty((1, 2), dtype=torch.float32, device="cuda:0")
    lo = torch.empty((1, 16), dtype=torch.int16, device="cuda:0")
    assert bd.svdq_quantize_act(cfg, 0, x.data_ptr() or c.data_ptr(), si, l1, 1.0, c, s, lo) == 0

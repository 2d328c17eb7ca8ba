"""GPU parity of svdq_gemm_w4a4_packed_quantize_next, the MLP pair with fc2's activation
kernel fused into fc1's GEMM epilogue: its packed codes, scale words and fp32 scales are
bit-identical to fc1's packed GEMM (bf16 out) followed by svdq_quantize_act_packed, and
its lora_act lies within the fp32 summation bound of the oracle's down-projection of the
same bf16 intermediate (bit-equal to it wherever that bound reaches no bf16 rounding
boundary), as the unfused activation kernel's does.  Shapes cover ragged token counts, fc1 widths that end in a
partial 192-column tile, GELU on and off, next ranks 0 to 128, and the MLP end to end
against the oracle chain."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.construct import bf16_from_f64_vec

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _fc1(rng, M, K1, N1, r1):
    x = synth.random_bf16(rng, (M, K1), 1.0)
    si1 = rng.uniform(0.5, 2.0, K1).astype(np.float32)
    l1 = synth.random_bf16(rng, (r1, K1), 0.05) if r1 else None
    l2 = synth.random_bf16(rng, (N1, r1), 0.1) if r1 else None
    cw = synth.random_packed_nibbles(rng, N1, K1)
    sw = rng.uniform(0.001, 0.05, (N1, K1 // 64)).astype(np.float32)
    b = synth.random_bf16(rng, (N1,), 0.3)
    return x, si1, l1, l2, cw, sw, b


@pytest.mark.parametrize("M,K1,N1,r1,r2,act", [
    (300, 256, 384, 16, 32, 1),     # ragged M, two full column tiles
    (300, 320, 448, 32, 32, 0),     # last column tile holds one 64-channel group
    (513, 192, 640, 0, 16, 1),      # three M tiles, no low-rank branch on fc1
    (64, 128, 192, 16, 0, 1),       # next rank 0: no down-projection
    (1000, 256, 1344, 32, 48, 1),   # seven column tiles, rank 48
    (1, 128, 576, 16, 16, 1),       # a single token
    (300, 128, 384, 16, 128, 1),    # the maximum next rank
    (260, 192, 448, 16, 128, 0),    # maximum rank with a partial last column tile
])
def test_fused_matches_unfused(M, K1, N1, r1, r2, act):
    rng = np.random.default_rng(1500 + M + N1 + r2)
    print(f"fused mlp M={M} K1={K1} N1={N1} r1={r1} r2={r2} act={act}", flush=True)
    x, si1, l1, l2, cw, sw, b = _fc1(rng, M, K1, N1, r1)
    si2 = rng.uniform(0.5, 2.0, N1).astype(np.float32)
    si2[5] = 0.02                                   # an outlier channel of the intermediate
    nl1 = synth.random_bf16(rng, (r2, N1), 0.05) if r2 else None
    buf, _, lora = gu.quantize_packed(x, si1, l1)
    wp = gu.prepack(cw, sw, K1, N1)
    h = gu.gemm_packed(buf, wp, M, K1, N1, lora, l2, b, act=act, out_bf16=True)
    ub, us, ul = gu.quantize_packed(h, si2, nl1)
    fb, fs, fl = gu.gemm_packed_quantize_next(buf, wp, M, K1, N1, lora, l2, b, act, si2, nl1)
    torch.cuda.synchronize()
    assert torch.equal(fb, ub), f"packed bytes differ in {int((fb != ub).sum())} places"
    assert torch.equal(fs.view(torch.int32), us.view(torch.int32)), "fp32 scales differ"
    if r2:
        hb = gu.host(h)
        ol = oracle.quant_act_int4(hb, si2, nl1)[2]
        gu.assert_lora_close(gu.host(fl), ol, hb, nl1)     # fused: per-tile partials
        gu.assert_lora_close(gu.host(ul), ol, hb, nl1)     # unfused: the activation kernel


def test_fused_without_scales_and_repeat():
    """next_act_scales NULL leaves the packed buffer unchanged, and a second call gives the
    same codes and, bit for bit, the same lora_act (fixed-order sum of the tiles' partials)."""
    M, K1, N1, r1, r2 = 260, 192, 384, 16, 32
    rng = np.random.default_rng(1520)
    x, si1, l1, l2, cw, sw, b = _fc1(rng, M, K1, N1, r1)
    si2 = rng.uniform(0.5, 2.0, N1).astype(np.float32)
    nl1 = synth.random_bf16(rng, (r2, N1), 0.05)
    buf, _, lora = gu.quantize_packed(x, si1, l1)
    wp = gu.prepack(cw, sw, K1, N1)
    b1, s1, l1o = gu.gemm_packed_quantize_next(buf, wp, M, K1, N1, lora, l2, b, 1, si2, nl1)
    b2, s2, l2o = gu.gemm_packed_quantize_next(buf, wp, M, K1, N1, lora, l2, b, 1, si2, nl1,
                                               with_scales=False)
    torch.cuda.synchronize()
    assert s2 is None and torch.equal(b1, b2)
    assert torch.equal(l1o, l2o), "lora_act differs between two calls"


@pytest.mark.parametrize("M,K1,N1,N2,r", [(300, 256, 448, 200, 16), (700, 192, 768, 384, 32)])
def test_fused_mlp_end_to_end(M, K1, N1, N2, r):
    """x -> fc1 (GELU) with fused fc2 quantization -> fc2, against the oracle chain
    fc1 -> GELU -> bf16 -> activation stage -> fc2 (relative Frobenius <= 1e-3)."""
    rng = np.random.default_rng(1530 + M)
    print(f"fused mlp end to end M={M} K1={K1} N1={N1} N2={N2} r={r}", flush=True)
    x, si1, l1, l2, cw, sw, b = _fc1(rng, M, K1, N1, r)
    si2 = rng.uniform(0.5, 2.0, N1).astype(np.float32)
    nl1 = synth.random_bf16(rng, (r, N1), 0.05)
    nl2 = synth.random_bf16(rng, (N2, r), 0.1)
    cw2 = synth.random_packed_nibbles(rng, N2, N1)
    sw2 = rng.uniform(0.001, 0.05, (N2, N1 // 64)).astype(np.float32)
    b2 = synth.random_bf16(rng, (N2,), 0.3)
    buf, _, lora = gu.quantize_packed(x, si1, l1)
    fb, _, fl = gu.gemm_packed_quantize_next(buf, gu.prepack(cw, sw, K1, N1), M, K1, N1, lora,
                                             l2, b, 1, si2, nl1)
    y = gu.host(gu.gemm_packed(fb, gu.prepack(cw2, sw2, N1, N2), M, N1, N2, fl, nl2, b2))
    oc, os_, ol = oracle.quant_act_int4(x, si1, l1)
    h = bf16_from_f64_vec(oracle.gemm_w4a4_int4(oc, os_, cw, sw, ol, l2, b, act=1))
    qc, qs, ql = oracle.quant_act_int4(h, si2, nl1)
    ref = oracle.gemm_w4a4_int4(qc, qs, cw2, sw2, ql, nl2, b2)
    e = gu.rel_fro(y, ref)
    print(f"fused mlp end-to-end rel_fro={e:.3e}")
    assert e <= 1e-3

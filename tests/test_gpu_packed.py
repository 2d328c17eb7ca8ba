"""GPU parity of the packed INT4 path (FP6 MFMA GEMM on MFMA-ready operands) against the
CPU oracle.

* svdq_gemm_w4a4_packed, fed the oracle-format operands through svdq_pack_act and
  svdq_prepack_weight, on shapes spanning several 256x192 tiles, ragged M and N, K from one
  group to 16, fewer groups than pipeline stages, ranks 0..128, bias, GELU and both output
  types, and the K split of a nearly empty last round of tiles (fp32 output).  Bar: relative
  Frobenius error <= 1e-3 of the oracle's fp64 result (fp32 output);
  bf16 output within one bf16 ulp (plus 2^-16 of the largest magnitude), >= 99% equal to
  the oracle rounded to bf16.
* svdq_prepack_l1: the reordered low-rank factor against the layout written out on the host.
* svdq_quantize_act_packed: the codes read back from the packed buffer, the fp32 scales and
  lora_act equal svdq_quantize_act's and the oracle's bit for bit (lora_act within its fp32
  bound); the scale words are the bf16 hi/lo split of the scales; padding rows are zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


def _inputs(rng, M, N, K, r, bias=True):
    ca, cw = synth.random_packed_nibbles(rng, M, K), synth.random_packed_nibbles(rng, N, K)
    sa = rng.uniform(0.01, 1.0, (M, K // 64)).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    lora = synth.random_bf16(rng, (M, r), 1.0) if r else None
    l2 = synth.random_bf16(rng, (N, r), 0.1) if r else None
    b = synth.random_bf16(rng, (N,), 0.3) if bias else None
    return ca, sa, cw, sw, lora, l2, b


@pytest.mark.parametrize("M,N,K,r,bias,act", [
    (1, 32, 64, 0, False, 0), (5, 96, 128, 16, True, 0), (257, 200, 192, 32, True, 0),
    (300, 384, 256, 16, True, 1), (64, 128, 320, 128, False, 1), (33, 17, 1024, 0, True, 0),
    (520, 400, 512, 32, True, 0), (256, 192, 384, 48, True, 0), (700, 390, 448, 16, False, 1),
])
def test_packed_gemm_shapes(M, N, K, r, bias, act):
    rng = np.random.default_rng(700 + M + N + K + r)
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r, bias)
    print(f"packed gemm M={M} N={N} K={K} r={r} bias={bias} act={act}", flush=True)
    ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw, lora, l2, b, act)
    packed = gu.prepack(cw, sw, K, N)
    y = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, act))
    e = gu.rel_fro(y, ref)
    assert e <= 1e-3, e
    assert e <= 1e-4, f"unexpectedly far from the oracle: {e}"
    cond = gu.int4_cond(ca, sa, cw, sw, lora, l2, b)
    gu.assert_f32_within(y, ref, cond, gu.int4_nround(K, r), gelu=act == 1)
    yb = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, act, out_bf16=True))
    gu.assert_bf16_close(yb, ref, cond, gu.int4_nround(K, r), gelu=act == 1)


def test_packed_gemm_unaligned_output_rows():
    # N * 2 bytes not a multiple of 16: the element-wise store path
    rng = np.random.default_rng(703)
    M, N, K, r = 130, 203, 192, 16
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r)
    ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw, lora, l2, b)
    packed = gu.prepack(cw, sw, K, N)
    cond = gu.int4_cond(ca, sa, cw, sw, lora, l2, b)
    yb = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, out_bf16=True))
    gu.assert_bf16_close(yb, ref, cond, gu.int4_nround(K, r))
    y = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b))
    assert gu.rel_fro(y, ref) <= 1e-4
    gu.assert_f32_within(y, ref, cond, gu.int4_nround(K, r))


def test_packed_extreme_codes():
    # all activation codes 7 / -7, weight codes -8 (largest magnitudes, both signs)
    M, N, K = 70, 130, 256
    for abyte in (0x77, 0x99):
        ca = np.full((M, K // 2), abyte, np.uint8)
        cw = np.full((N, K // 2), 0x88, np.uint8)
        sa = np.full((M, K // 64), 0.5, np.float32)
        sw = np.full((N, K // 64), 0.25, np.float32)
        ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw)
        y = gu.host(gu.gemm_prepacked(ca, sa, gu.prepack(cw, sw, K, N), N))
        assert gu.rel_fro(y, ref) <= 1e-4


def test_packed_matches_reference_kernel_and_is_deterministic():
    rng = np.random.default_rng(701)
    M, N, K, r = 600, 576, 768, 32
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r)
    packed = gu.prepack(cw, sw, K, N)
    y1 = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b))
    y2 = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b))
    assert np.array_equal(y1, y2)
    y0 = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b))
    assert gu.rel_fro(y1, y0) <= 1e-4


@pytest.mark.parametrize("M,N", [(4352, 3072), (4300, 2998)])
def test_packed_gemm_k_split_last_round(M, N):
    """17 x 16 output tiles on a 256-CU GPU: with a workspace, the last round's 16 tiles run
    as 8 K splits each, summed in a fixed order by a second kernel.  The whole output against
    the unsplit call (the same products in another fp32 order) and the nibble-operand kernel
    (a different code path, itself checked against the oracle); samples against the oracle
    within the fp32 error bound (rows of the split tiles and of whole tiles); two calls
    bit-identical; bf16 output (no split) at the samples."""
    K, r = 1024, 32
    rng = np.random.default_rng(710 + M + N)
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r)
    print(f"packed gemm K split M={M} N={N} K={K} r={r}", flush=True)
    assert gu.split_workspace_bytes(M, K, N) > 0, "this shape is expected to split"
    packed = gu.prepack(cw, sw, K, N)
    ap = gu.pack_act(ca, sa, K)
    y = gu.host(gu.gemm_packed(ap, packed, M, K, N, lora, l2, b, split=True))
    y_again = gu.host(gu.gemm_packed(ap, packed, M, K, N, lora, l2, b, split=True))
    assert np.array_equal(y.view(np.uint32), y_again.view(np.uint32)), "K split not reproducible"
    y1 = gu.host(gu.gemm_packed(ap, packed, M, K, N, lora, l2, b))
    assert np.array_equal(y[:4096], y1[:4096]), "whole tiles differ between the two calls"
    assert gu.rel_fro(y, y1) <= 1e-6
    y0 = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b))
    assert gu.rel_fro(y, y0) <= 1e-5
    mi = np.concatenate([rng.integers(4096, M, 600), rng.integers(0, 4096, 200)])
    ni = rng.integers(0, N, mi.shape[0])
    ref = oracle.gemm_w4a4_int4_at(mi, ni, ca, sa, cw, sw, lora, l2, b)
    assert gu.rel_fro(y[mi, ni], ref) <= 1e-5
    cond = gu.int4_cond(ca, sa, cw, sw, lora, l2, b, mi, ni)
    gu.assert_f32_within(y[mi, ni], ref, cond, gu.int4_nround(K, r))
    yb = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, out_bf16=True))
    gu.assert_bf16_close(yb[mi, ni], ref, cond, gu.int4_nround(K, r))


@pytest.mark.parametrize("M,K,r", [(1, 64, 0), (100, 192, 16), (256, 512, 32), (300, 1024, 32),
                                   (513, 320, 48), (40, 3072, 128)])
def test_quantize_packed_bit_exact(M, K, r):
    rng = np.random.default_rng(900 + M + K + r)
    x = synth.random_bf16(rng, (M, K), 1.0)
    x[:, rng.integers(0, K, max(1, K // 50))] = synth.random_bf16(rng, (M, max(1, K // 50)), 30.0)
    si = rng.uniform(0.25, 4.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05) if r else None
    print(f"quantize packed M={M} K={K} r={r}", flush=True)
    buf, scales, lora = gu.quantize_packed(x, si, l1)
    codes_n, scales_n, lora_n = gu.quantize(x, si, l1)
    torch.cuda.synchronize()
    oc, os_, ol = oracle.quant_act_int4(x, si, l1)
    q, words, canonical = gu.decode_act_packed(gu.host(buf), M, K)
    assert canonical
    assert np.array_equal(q[:M], oracle.unpack_int4(oc).astype(np.int64)), "codes differ"
    assert not q[M:].any() and not words[M:].any(), "padding rows not zero"
    gs = gu.host(scales)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"
    assert np.array_equal(gs.view(np.uint32), gu.host(scales_n).view(np.uint32))
    assert np.array_equal(words[:M], gu.split_words(os_)), "scale words differ"
    if r:
        assert np.array_equal(gu.host(lora), gu.host(lora_n))
        gu.assert_lora_close(gu.host(lora), ol, x, l1)
    # the packed buffer from nibbles is the same bytes
    assert torch.equal(gu.pack_act(codes_n, scales_n, K), buf)


@pytest.mark.parametrize("K,r", [(64, 16), (192, 32), (3072, 32), (320, 128)])
def test_prepack_l1_layout(K, r):
    """svdq_prepack_l1 against the layout written out on the host: unit (c, b, t), lane L
    holds L1[16 b + L % 16][128 c + 32 (L / 16) + 8 t .. + 8], zeros past K."""
    rng = np.random.default_rng(910 + K + r)
    l1 = synth.random_bf16(rng, (r, K), 0.05)
    got = gu.host(gu.prepack_l1(l1, K)).view(np.uint16)
    nc = (K + 127) // 128
    padded = np.zeros((r, nc * 128), np.uint16)
    padded[:, :K] = l1
    want = np.empty((nc, r // 16, 4, 64, 8), np.uint16)
    for c in range(nc):
        for b in range(r // 16):
            for t in range(4):
                for L in range(64):
                    k = 128 * c + 32 * (L // 16) + 8 * t
                    want[c, b, t, L] = padded[16 * b + L % 16, k:k + 8]
    assert np.array_equal(got, want.reshape(-1))


def test_quantize_packed_without_scales():
    rng = np.random.default_rng(905)
    M, K = 77, 256
    x = synth.random_bf16(rng, (M, K), 1.0)
    si = rng.uniform(0.5, 2.0, K).astype(np.float32)
    buf, _, _ = gu.quantize_packed(x, si, None, with_scales=False)
    oc, os_, _ = oracle.quant_act_int4(x, si, None)
    q, words, _ = gu.decode_act_packed(gu.host(buf), M, K)
    assert np.array_equal(q[:M], oracle.unpack_int4(oc).astype(np.int64))
    assert np.array_equal(words[:M], gu.split_words(os_))


def test_quantize_packed_then_gemm_end_to_end():
    rng = np.random.default_rng(906)
    M, N, K, r = 300, 392, 448, 32
    x = synth.random_bf16(rng, (M, K), 1.0)
    si = rng.uniform(0.5, 2.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05)
    cw = synth.random_packed_nibbles(rng, N, K)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    l2 = synth.random_bf16(rng, (N, r), 0.1)
    b = synth.random_bf16(rng, (N,), 0.3)
    oc, os_, ol = oracle.quant_act_int4(x, si, l1)
    ref = oracle.gemm_w4a4_int4(oc, os_, cw, sw, ol, l2, b)
    buf, _, lora = gu.quantize_packed(x, si, l1)
    y = gu.host(gu.gemm_packed(buf, gu.prepack(cw, sw, K, N), M, K, N, lora, l2, b))
    assert gu.rel_fro(y, ref) <= 1e-3


def test_tiny_workload_packed_end_to_end():
    """The tiny workload (256 tokens, K = N = 512, rank 16, no bias) through the calls the
    benchmark times: svdq_prepack_l1 + svdq_quantize_act_packed (codes read back from the
    packed buffer and fp32 scales bit-exact, lora_act within its fp32 bound), then
    svdq_prepack_weight + svdq_gemm_w4a4_packed (fp32 output within the fp32 error bound of
    the oracle element by element and 1e-3 relative Frobenius; bf16 output among the bf16
    roundings of that bound)."""
    from oracle.construct import build_workload
    d, (L,) = build_workload(synth.WORKLOADS[0])
    M, K = d.x_bf16.shape
    N, r = L["wcodes"].shape[0], L["rank"]
    print(f"tiny workload packed M={M} K={K} N={N} r={r}", flush=True)
    buf, scales, lora = gu.quantize_packed(d.x_bf16, L["smooth_inv"], L["l1"], N=N)
    torch.cuda.synchronize()
    oc, os_, ol = oracle.quant_act_int4(d.x_bf16, L["smooth_inv"], L["l1"])
    q, words, canonical = gu.decode_act_packed(gu.host(buf), M, K)
    assert canonical
    assert np.array_equal(q[:M], oracle.unpack_int4(oc).astype(np.int64)), "codes differ"
    assert np.array_equal(gu.host(scales).view(np.uint32), os_.view(np.uint32)), "scales differ"
    gu.assert_lora_close(gu.host(lora), ol, d.x_bf16, L["l1"])
    wp = gu.prepack(L["wcodes"], L["wscales"], K, N)
    ref = oracle.gemm_w4a4_int4(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], None)
    cond = gu.int4_cond(oc, os_, L["wcodes"], L["wscales"], ol, L["l2"], None)
    # GEMM on the oracle's activation outputs: element-wise bound
    y = gu.host(gu.gemm_packed(gu.pack_act(oc, os_, K), wp, M, K, N, ol, L["l2"], None))
    gu.assert_f32_within(y, ref, cond, gu.int4_nround(K, r))
    yb = gu.host(gu.gemm_packed(gu.pack_act(oc, os_, K), wp, M, K, N, ol, L["l2"], None, out_bf16=True))
    gu.assert_bf16_close(yb, ref, cond, gu.int4_nround(K, r))
    # end to end from the GPU's own activation stage
    ye = gu.host(gu.gemm_packed(buf, wp, M, K, N, lora, L["l2"], None))
    assert gu.rel_fro(ye, ref) <= 1e-3
    exact = oracle.bf16_to_f64(d.x_bf16) @ d.w.T   # and the method did its job
    assert gu.rel_fro(ye, exact) < 0.2

"""GPU parity of the prepacked INT4 GEMM (FP6 MFMA main loop) against the CPU oracle, on
shapes spanning several 256x192 tiles, ragged M and N, K of 1..5 correction windows (partial
last window included), ranks 0..128, bias, GELU and both output types.
Bar: relative Frobenius error <= 1e-3 of the oracle's fp64 result (fp32 output); bf16 output
within one bf16 ulp (plus 2^-16 of the largest magnitude), >= 99% equal to the oracle
rounded to bf16."""
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
    (520, 400, 512, 32, True, 0),
])
def test_prepacked_gemm_shapes(M, N, K, r, bias, act):
    rng = np.random.default_rng(700 + M + N + K + r)
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r, bias)
    ref = oracle.gemm_w4a4_int4(ca, sa, cw, sw, lora, l2, b, act)
    packed = gu.prepack(cw, sw, K, N)
    y = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, act))
    e = gu.rel_fro(y, ref)
    assert e <= 1e-3, e
    assert e <= 1e-4, f"unexpectedly far from the oracle: {e}"
    yb = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b, act, out_bf16=True))
    gu.assert_bf16_close(yb, ref)


def test_prepacked_extreme_codes():
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


def test_prepacked_matches_reference_kernel_and_is_deterministic():
    rng = np.random.default_rng(701)
    M, N, K, r = 600, 576, 768, 32
    ca, sa, cw, sw, lora, l2, b = _inputs(rng, M, N, K, r)
    packed = gu.prepack(cw, sw, K, N)
    y1 = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b))
    y2 = gu.host(gu.gemm_prepacked(ca, sa, packed, N, lora, l2, b))
    assert np.array_equal(y1, y2)
    y0 = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b))
    assert gu.rel_fro(y1, y0) <= 1e-4

"""GPU parity of the NVFP4 path and the AWQ W4A16 GEMV against the CPU oracle (small and
ragged shapes).  Bar: codes / E4M3 scales bit-exact; lora_act within 1 bf16 ulp; outputs
within relative Frobenius 1e-3 of the oracle's fp64 result."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.construct import bf16_from_f64_vec

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")


@pytest.mark.parametrize("M,K,r", [(1, 64, 0), (19, 256, 16), (128, 512, 32), (300, 192, 48)])
def test_quant_nvfp4_shapes(M, K, r):
    rng = np.random.default_rng(400 + M + K + r)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, 3, replace=False)] *= 50
    if M > 2:
        x[1, :16] = 0.0
        x[2, :] *= 1e-6          # many zero / subnormal block scales
    xb = synth.f32_to_bf16_bits(x)
    si = rng.uniform(0.1, 2.0, K).astype(np.float32)
    xhat = synth.bf16_bits_to_f32(xb) * si[None, :]
    S = np.float32(np.max(np.abs(xhat)) / np.float32(2688))
    l1 = synth.random_bf16(rng, (r, K), 0.05) if r else None
    for SS in (S, np.float32(S * 4), np.float32(S / 64)):   # also saturating / tiny scales
        codes, scales, lora = gu.quantize(xb, si, l1, "nvfp4", float(SS))
        oc, os_, ol = oracle.quant_act_nvfp4(xb, si, SS, l1)
        assert np.array_equal(gu.host(codes), oc)
        assert np.array_equal(gu.host(scales), os_)
        if r:
            gu.assert_lora_close(gu.host(lora), ol, xb, l1)


# K a multiple of 256 takes the fast kernel (two, three and four 256-channel stages over
# several 256 x 192 tiles with ragged row and column tails); other K the reference kernel.
@pytest.mark.parametrize("M,N,K,r,bias,act", [
    (1, 128, 64, 0, False, 0), (7, 96, 192, 16, True, 0), (130, 260, 512, 32, True, 1),
    (300, 400, 1024, 32, True, 0), (513, 200, 640, 16, False, 1), (257, 193, 320, 0, True, 0),
    (70, 500, 768, 16, True, 1), (1, 20, 256, 0, False, 0),
])
def test_gemm_nvfp4_shapes(M, N, K, r, bias, act):
    rng = np.random.default_rng(500 + M + N + K)
    ca, cw = synth.random_packed_nibbles(rng, M, K), synth.random_packed_nibbles(rng, N, K)
    sa = rng.integers(0, 0x7F, size=(M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)
    Sa, Sw = np.float32(0.003), np.float32(0.0007)
    lora = synth.random_bf16(rng, (M, r), 1.0) if r else None
    l2 = synth.random_bf16(rng, (N, r), 0.1) if r else None
    b = synth.random_bf16(rng, (N,), 0.3) if bias else None
    ref = oracle.gemm_w4a4_nvfp4(ca, sa, Sa, cw, sw, Sw, lora, l2, b, act)
    y = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b, act, precision="nvfp4", Sa=Sa, Sw=Sw))
    e = gu.rel_fro(y, ref)
    assert e <= 1e-3, e
    assert e <= 1e-5, e
    yb = gu.host(gu.gemm(ca, sa, cw, sw, lora, l2, b, act, True, "nvfp4", Sa, Sw))
    gu.assert_bf16_close(yb, ref)


def test_gemm_nvfp4_unaligned_scales():
    """E4M3 scale arrays that are not 16-byte aligned are accepted (they take the reference
    kernel)."""
    M, N, K, r = 70, 130, 256, 16
    rng = np.random.default_rng(520)
    ca, cw = synth.random_packed_nibbles(rng, M, K), synth.random_packed_nibbles(rng, N, K)
    sa = rng.integers(0, 0x7F, size=(M, K // 16)).astype(np.uint8)
    sw = rng.integers(0, 0x7F, size=(N, K // 16)).astype(np.uint8)
    Sa, Sw = np.float32(0.002), np.float32(0.001)
    lora, l2 = synth.random_bf16(rng, (M, r), 1.0), synth.random_bf16(rng, (N, r), 0.1)
    ref = oracle.gemm_w4a4_nvfp4(ca, sa, Sa, cw, sw, Sw, lora, l2, None, 0)

    def shifted(a):
        buf = torch.zeros(a.size + 1, dtype=torch.uint8, device="cuda:0")
        buf[1:] = gu.dev(a).reshape(-1)
        return buf[1:].view(a.shape)

    y = gu.host(gu.gemm(ca, shifted(sa), cw, shifted(sw), lora, l2, None, 0, precision="nvfp4",
                        Sa=Sa, Sw=Sw))
    assert gu.rel_fro(y, ref) <= 1e-5


# M <= 4 with K a multiple of 512 up to 4096 runs the MFMA kernel, everything else the
# reference kernel; N not a multiple of 16 leaves a partial column tile; N = 25000 at
# K = 3072 needs more workgroups than fit in LDS at once (several columns runs per CU)
@pytest.mark.parametrize("M,N,K", [
    (1, 64, 64), (2, 130, 3072), (5, 33, 512), (9, 100, 256), (3, 70, 768), (4, 96, 1024),
    (2, 64, 1536), (1, 40, 2048), (4, 50, 4096), (6, 50, 4096), (2, 32, 1152), (2, 48, 4160),
    (13, 200, 3072), (1, 25000, 3072), (2, 1000, 512),
])
def test_awq_shapes(M, N, K):
    rng = np.random.default_rng(600 + M + N + K)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, sc, z = oracle.awq_quant_weight(w)
    x = synth.random_bf16(rng, (M, K), 1.0)
    b = synth.random_bf16(rng, (N,), 0.1)
    for bias in (None, b):
        ref = oracle.awq_gemv(x, q, sc, z, bias)
        y = gu.host(gu.awq(x, q, sc, z, bias))
        assert gu.rel_fro(y, ref) <= 1e-3
        assert gu.rel_fro(y, ref) <= 1e-5
        yb = gu.host(gu.awq(x, q, sc, z, bias, out_bf16=True))
        gu.assert_bf16_close(yb, ref)


def test_awq_unaligned_scales():
    """Scales and zeros at 2-byte (not 16-byte) aligned addresses are accepted (they take
    the reference kernel); results within the same bound as aligned ones."""
    M, N, K = 2, 70, 3072
    rng = np.random.default_rng(611)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, sc, z = oracle.awq_quant_weight(w)
    x = synth.random_bf16(rng, (M, K), 1.0)
    ref = oracle.awq_gemv(x, q, sc, z, None)

    def shifted(a):
        buf = torch.zeros(a.size + 1, dtype=torch.int16, device="cuda:0")
        buf[1:] = gu.dev(a).reshape(-1)
        return buf[1:].view(a.shape)

    out = gu.empty((M, N), np.float32)
    gu.bd.awq_gemm_w4a16(M, K, N, 64, gu.dev(x), gu.dev(q), shifted(sc), shifted(z), None,
                         gu.bd.SVDQ_DT_F32, out)
    y = gu.host(out)
    assert gu.rel_fro(y, ref) <= 1e-5
    assert gu.rel_fro(gu.host(gu.awq(x, q, sc, z, None)), ref) <= 1e-5

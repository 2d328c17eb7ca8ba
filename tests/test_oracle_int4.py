"""Pins of the oracle's INT4 activation stage against facts other than itself.

Definition under test (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers",
技术细节 1 steps 1, 3, 4; 64-channel groups, scale absmax/7 in fp32, round half to even,
clamp to [-8, 7], two's-complement nibbles with the even channel in the low nibble).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import bruteforce as bf
from oracle.construct import bf16_from_f64_vec


def _x(rng, M, K, std=1.0):
    return synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * std).astype(np.float32))


def test_lossless_roundtrip_powers_of_two():
    # x = 2^e * c with integer c in [-7, 7] and |c| = 7 present in every group:
    # the scale must come back as exactly 2^e and the codes as c.
    rng = np.random.default_rng(1)
    M, K = 8, 256
    c = rng.integers(-7, 8, size=(M, K))
    c[:, ::64] = 7 * np.where(rng.random((M, K // 64)) < 0.5, 1, -1)
    e = rng.integers(-20, 10, size=(M, K // 64))
    x = c * np.ldexp(1.0, np.repeat(e, 64, axis=1))
    xb = synth.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(synth.bf16_bits_to_f32(xb), x.astype(np.float32))
    codes, scales, _ = oracle.quant_act_int4(xb, np.ones(K, np.float32))
    assert np.array_equal(scales, np.ldexp(1.0, e).astype(np.float32))
    assert np.array_equal(oracle.unpack_int4(codes), c.astype(np.int8))


def test_power_of_two_equivariance_and_sign_symmetry():
    rng = np.random.default_rng(2)
    M, K = 16, 512
    xb = _x(rng, M, K)
    si = (rng.uniform(0.1, 2.0, K)).astype(np.float32)
    codes, scales, _ = oracle.quant_act_int4(xb, si)
    for p in (-3, 5):
        x2 = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(xb) * np.float32(2.0 ** p))
        c2, s2, _ = oracle.quant_act_int4(x2, si)
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, scales * np.float32(2.0 ** p))
    xn = xb ^ np.uint16(0x8000)
    cn, sn, _ = oracle.quant_act_int4(xn, si)
    assert np.array_equal(sn, scales)
    assert np.array_equal(oracle.unpack_int4(cn).astype(np.int16),
                          -oracle.unpack_int4(codes).astype(np.int16))


def test_matches_exhaustive_nearest_search():
    rng = np.random.default_rng(3)
    M, K = 64, 512
    xb = _x(rng, M, K)
    xb[:, 7] = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(xb[:, 7]) * 30)
    si = rng.uniform(0.05, 3.0, K).astype(np.float32)
    codes, scales, _ = oracle.quant_act_int4(xb, si)
    xhat = synth.bf16_bits_to_f32(xb) * si[None, :]
    s_rep = np.repeat(scales, 64, axis=1)
    ref, near_tie = bf.nearest_int4(xhat, s_rep)
    got = oracle.unpack_int4(codes)
    agree = got == ref
    assert np.all(agree | near_tie)
    # where they may differ, the fp32-division definition decides
    q = np.clip(np.rint((xhat / s_rep).astype(np.float32)), -8, 7).astype(np.int8)
    assert np.array_equal(got[near_tie], q[near_tie])
    # scale: exactly fp32(absmax / 7)
    amax = np.abs(xhat).reshape(M, K // 64, 64).max(axis=2)
    assert np.array_equal(scales, (amax / np.float32(7.0)).astype(np.float32))


def test_matches_torch_round_on_fp32_quotients():
    rng = np.random.default_rng(4)
    M, K = 32, 1024
    xb = _x(rng, M, K, 3.0)
    si = rng.uniform(0.1, 1.0, K).astype(np.float32)
    codes, scales, _ = oracle.quant_act_int4(xb, si)
    xt = torch.from_numpy(synth.bf16_bits_to_f32(xb)) * torch.from_numpy(si)[None, :]
    st = torch.from_numpy(scales).repeat_interleave(64, dim=1)
    qt = torch.clamp(torch.round(xt / st), -8, 7).to(torch.int8).numpy()
    assert np.array_equal(oracle.unpack_int4(codes), qt)


def test_codes_never_minus_eight_and_zero_group():
    rng = np.random.default_rng(5)
    M, K = 64, 512
    xb = _x(rng, M, K, 10.0)
    xb[3, 64:128] = 0
    xb[5, 0:64] = 0x8000  # negative zeros
    codes, scales, _ = oracle.quant_act_int4(xb, np.ones(K, np.float32))
    q = oracle.unpack_int4(codes)
    assert q.min() >= -7 and q.max() <= 7
    assert scales[3, 1] == 0 and np.all(q[3, 64:128] == 0)
    assert scales[5, 0] == 0 and np.all(q[5, 0:64] == 0)


def test_packing_layout_hand_case():
    # one row, one group: codes 0..7 then -8.. appear in known nibbles
    K = 64
    vals = np.zeros(K, np.float32)
    vals[0], vals[1], vals[2], vals[3] = 7.0, -7.0, 1.0, -1.0
    xb = synth.f32_to_bf16_bits(vals[None, :])
    codes, scales, _ = oracle.quant_act_int4(xb, np.ones(K, np.float32))
    assert scales[0, 0] == np.float32(1.0)
    assert codes[0, 0] == 0x97  # low nibble 7 (k=0), high nibble -7 = 0x9 (k=1)
    assert codes[0, 1] == 0xF1  # low nibble 1 (k=2), high nibble -1 = 0xF (k=3)
    assert np.all(codes[0, 2:] == 0)


def test_lowrank_down_single_rounding():
    rng = np.random.default_rng(6)
    M, K, r = 16, 512, 8
    xb = _x(rng, M, K)
    l1 = _x(rng, r, K, 0.05)
    _, _, lora = oracle.quant_act_int4(xb, np.ones(K, np.float32), l1)
    ref = bf.lowrank_down_f64(xb, l1)
    assert np.array_equal(lora, bf16_from_f64_vec(ref))
    # and against torch: fp64 matmul rounded through fp32 to bf16 agrees up to 1 ulp
    t = (torch.from_numpy(oracle.bf16_to_f64(xb)) @ torch.from_numpy(oracle.bf16_to_f64(l1)).T)
    tb = t.to(torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.max(np.abs(tb.astype(np.int32) - lora.astype(np.int32))) <= 1


def test_bf16_rounding_helpers_agree():
    rng = np.random.default_rng(7)
    d = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000),
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, 3.0e38, 1e-40]])
    a = oracle.bf16_from_f64(d)
    b = bf16_from_f64_vec(d)
    assert np.array_equal(a, b)
    # ties to even: 1 + 2^-8 -> 1.0 ; 1 + 3*2^-8 -> 1 + 2^-6 (even mantissa)
    assert a[-4] == 0x3F80 and a[-3] == 0x3F82
    # for fp32-representable inputs it is torch's fp32 -> bf16 cast
    f = rng.standard_normal(4000).astype(np.float32) * np.float32(1e3)
    tb = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_from_f64_vec(f.astype(np.float64)), tb)


@pytest.mark.parametrize("M,K", [(1, 64), (3, 192)])
def test_small_shapes(M, K):
    rng = np.random.default_rng(8)
    xb = _x(rng, M, K)
    codes, scales, lora = oracle.quant_act_int4(xb, np.ones(K, np.float32))
    assert codes.shape == (M, K // 2) and scales.shape == (M, K // 64) and lora.shape == (M, 0)

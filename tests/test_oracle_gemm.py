"""Pins of the oracle's INT4 W4A4 GEMM (per-group integer dots, scales, low-rank
up-projection, bias, GELU) against independent formulations and closed forms.

Definition (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到 Diffusers", 技术细节 1
step 4: the low-rank up-projection is fused into the 4-bit compute kernel):
    Y[m,n] = sum_g sa[m,g] sw[n,g] sum_{k in g} qa[m,k] qw[n,k]
             + sum_j lora[m,j] l2[n,j] + b[n]        (optionally GELU-tanh).
"""
import numpy as np
import torch

import oracle
import synth
from oracle import bruteforce as bf


def _rand_int4(rng, R, K):
    return synth.random_packed_nibbles(rng, R, K)


def _inputs(rng, M, N, K, r, bias=True):
    ca, cw = _rand_int4(rng, M, K), _rand_int4(rng, N, K)
    sa = rng.uniform(0.01, 1.0, (M, K // 64)).astype(np.float32)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    lora = synth.random_bf16(rng, (M, r), 1.0)
    l2 = synth.random_bf16(rng, (N, r), 0.1)
    b = synth.random_bf16(rng, (N,), 0.1) if bias else None
    return ca, sa, cw, sw, lora, l2, b


def test_group_dots_equal_dequantize_then_matmul():
    rng = np.random.default_rng(10)
    M, N, K, r = 24, 40, 320, 8
    args = _inputs(rng, M, N, K, r)
    Y = oracle.gemm_w4a4_int4(*args)
    Yb = bf.gemm_dequant_int4(*args)
    assert np.max(np.abs(Y - Yb)) <= 1e-12 * np.max(np.abs(Yb))


def test_rank_zero_no_bias_is_plain_w4a4():
    rng = np.random.default_rng(11)
    M, N, K = 8, 16, 128
    ca, sa, cw, sw, _, _, _ = _inputs(rng, M, N, K, 0, bias=False)
    Y = oracle.gemm_w4a4_int4(ca, sa, cw, sw)
    qa = oracle.unpack_int4(ca).astype(np.int64)
    qw = oracle.unpack_int4(cw).astype(np.int64)
    # textbook: per group integer matmul, then outer product of scales
    ref = np.zeros((M, N))
    for g in range(K // 64):
        D = qa[:, g * 64:(g + 1) * 64] @ qw[:, g * 64:(g + 1) * 64].T
        ref += np.outer(sa[:, g].astype(np.float64), sw[:, g].astype(np.float64)) * D
    assert np.allclose(Y, ref, rtol=1e-14, atol=0)


def test_all_sevens_closed_form():
    M, N, K = 3, 5, 192
    ca = np.full((M, K // 2), 0x77, np.uint8)
    cw = np.full((N, K // 2), 0x77, np.uint8)
    sa = np.full((M, K // 64), 0.5, np.float32)
    sw = np.full((N, K // 64), 0.25, np.float32)
    Y = oracle.gemm_w4a4_int4(ca, sa, cw, sw)
    assert np.all(Y == 3 * 64 * 49 * 0.5 * 0.25)
    # mixed signs: A = +7, W = -7 -> each group -3136
    cw2 = np.full((N, K // 2), 0x99, np.uint8)
    Y2 = oracle.gemm_w4a4_int4(ca, sa, cw2, sw)
    assert np.all(Y2 == -3 * 3136 * 0.125)


def test_k64_hand_case_transposition_sensitive():
    # one group, M=2, N=3, codes chosen so that A W^T != W A^T patterns
    K = 64
    qa = np.zeros((2, K), np.int64)
    qw = np.zeros((3, K), np.int64)
    qa[0, 0], qa[0, 1], qa[1, 2] = 1, 2, -3
    qw[0, 0], qw[1, 1], qw[2, 2], qw[2, 1] = 4, -5, 6, 7

    def pack(q):
        u = (q & 0xF).astype(np.uint8)
        return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)

    sa = np.array([[1.0], [2.0]], np.float32)
    sw = np.array([[1.0], [0.5], [0.25]], np.float32)
    lora = synth.f32_to_bf16_bits(np.array([[1.0], [0.0]], np.float32))
    l2 = synth.f32_to_bf16_bits(np.array([[10.0], [20.0], [30.0]], np.float32))
    b = synth.f32_to_bf16_bits(np.array([0.5, 0.25, 0.125], np.float32))
    Y = oracle.gemm_w4a4_int4(pack(qa), sa, pack(qw), sw, lora, l2, b)
    # hand: D = qa qw^T = [[4, -10, 14], [0, 0, -18]]
    expect = np.array([[4 * 1 + 10 + 0.5, -10 * 0.5 + 20 + 0.25, 14 * 0.25 + 30 + 0.125],
                       [0 + 0.5, 0 + 0.25, -18 * 2 * 0.25 + 0.125]])
    assert np.array_equal(Y, expect)


def test_gelu_matches_torch_fp64():
    y = np.linspace(-8, 8, 2001)
    g = oracle.gelu_tanh(y)
    t = torch.nn.functional.gelu(torch.from_numpy(y), approximate="tanh").numpy()
    assert np.max(np.abs(g - t)) <= 1e-15 * 8
    rng = np.random.default_rng(12)
    args = _inputs(rng, 4, 6, 128, 4)
    Y0 = oracle.gemm_w4a4_int4(*args, act=0)
    Y1 = oracle.gemm_w4a4_int4(*args, act=1)
    assert np.allclose(Y1, oracle.gelu_tanh(Y0), rtol=0, atol=1e-15)


def test_sampled_outputs_match_full():
    rng = np.random.default_rng(13)
    M, N, K, r = 16, 24, 256, 4
    args = _inputs(rng, M, N, K, r)
    Y = oracle.gemm_w4a4_int4(*args)
    mi = rng.integers(0, M, 50)
    ni = rng.integers(0, N, 50)
    Ys = oracle.gemm_w4a4_int4_at(mi, ni, *args)
    assert np.array_equal(Ys, Y[mi, ni])

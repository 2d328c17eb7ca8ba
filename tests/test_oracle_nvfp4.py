"""Pins of the oracle's NVFP4 path (page "Hugging Face 把 Nunchaku 4-bit Diffusion 接到
Diffusers", 技术细节 3: svdq_w4a4 with precision nvfp4).  Format facts pinned here come
from the OCP 8-bit / 4-bit float definitions: E4M3 "FN" (bias 7, max 448, no infinities)
and E2M1 (0, 0.5, 1, 1.5, 2, 3, 4, 6), checked against torch's casts and exhaustive search.
"""
import numpy as np
import torch

import oracle
import synth
from oracle import bruteforce as bf


def _all_e4m3_values():
    b = np.arange(0, 0x7F, dtype=np.uint8)   # non-negative finite codes
    return b, oracle.e4m3_decode(b)


def test_e4m3_decode_matches_torch():
    b, v = _all_e4m3_values()
    t = torch.from_numpy(b.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(v, t)
    assert v.max() == 448.0 and v[1] == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast_below_448():
    rng = np.random.default_rng(20)
    x = np.concatenate([
        np.exp(rng.uniform(np.log(1e-4), np.log(448.0), 20000)),
        _all_e4m3_values()[1],
        (_all_e4m3_values()[1][:-1] + _all_e4m3_values()[1][1:]) / 2,   # exact ties
        [2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11],
    ]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got, ref)


def test_e4m3_saturates_and_exhaustive_nearest():
    assert oracle.e4m3_encode(np.float32([464.0, 500.0, 1e9]))[:].tolist() == [0x7E] * 3
    b, v = _all_e4m3_values()
    rng = np.random.default_rng(21)
    x = np.exp(rng.uniform(np.log(1e-4), np.log(448.0), 3000)).astype(np.float32)
    got = oracle.e4m3_decode(oracle.e4m3_encode(x))
    d = np.abs(x.astype(np.float64)[:, None] - v[None, :])
    best = v[np.argmin(d, axis=1)]
    tie = np.sort(d, axis=1)[:, 1] == np.min(d, axis=1)
    assert np.array_equal(got[~tie], best[~tie])


def test_e2m1_encode_exhaustive_ties_to_even():
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    assert np.array_equal(oracle.e2m1_decode(np.arange(8)), mags)
    assert np.array_equal(oracle.e2m1_decode(np.arange(8, 16)), -mags)
    pts = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.2, 0.3, 4.9, 5.1, 7.0, 100.0],
                   np.float32)
    exp = [0, 2, 2, 4, 4, 6, 6, 0, 1, 6, 7, 7, 7]
    assert oracle.e2m1_encode(pts).tolist() == exp
    assert oracle.e2m1_encode(-pts).tolist() == [e | 8 for e in exp]
    rng = np.random.default_rng(22)
    x = rng.uniform(-8, 8, 5000).astype(np.float32)
    c = oracle.e2m1_encode(x)
    v = oracle.e2m1_decode(c)
    d = np.abs(np.abs(x)[:, None].astype(np.float64) - mags[None, :])
    assert np.array_equal(np.abs(v), mags[np.argmin(d, axis=1)])
    assert np.all(np.signbit(x) == ((c & 8) > 0))


def test_nvfp4_block_roundtrip_on_grid():
    # values = e2m1 * sb * S with sb an E4M3 value and the block max = 6 * sb * S
    rng = np.random.default_rng(23)
    S = np.float32(0.125)
    R, K = 4, 64
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    codes = rng.integers(0, 16, size=(R, K)).astype(np.uint8)
    codes[:, ::16] = 7   # magnitude 6 in every block
    sbv = np.float32(2.0) ** rng.integers(-3, 4, size=(R, K // 16)).astype(np.float32)
    vals = np.where(codes & 8, -1, 1) * mags[codes & 7] * np.repeat(sbv, 16, axis=1) * S
    c, s = oracle.quant_rows_nvfp4(vals.astype(np.float32), S)
    assert np.array_equal(oracle.e4m3_decode(s.reshape(-1)).reshape(s.shape), sbv)
    u = oracle.unpack_u4(c)
    # -0 encodes as 0x8: compare values, not codes, for the zero magnitude
    assert np.array_equal(oracle.e2m1_decode(u.reshape(-1)).reshape(u.shape),
                          oracle.e2m1_decode(codes.reshape(-1)).reshape(codes.shape))


def test_nvfp4_gemm_equals_dequant_matmul():
    rng = np.random.default_rng(24)
    M, N, K, r = 8, 12, 128, 4
    ca, cw = synth.random_packed_nibbles(rng, M, K), synth.random_packed_nibbles(rng, N, K)
    sa = rng.integers(0x08, 0x60, size=(M, K // 16)).astype(np.uint8)
    sw = rng.integers(0x08, 0x60, size=(N, K // 16)).astype(np.uint8)
    Sa, Sw = np.float32(0.01), np.float32(0.003)
    lora = synth.random_bf16(rng, (M, r), 1.0)
    l2 = synth.random_bf16(rng, (N, r), 0.1)
    b = synth.random_bf16(rng, (N,), 0.1)
    Y = oracle.gemm_w4a4_nvfp4(ca, sa, Sa, cw, sw, Sw, lora, l2, b)
    Yb = bf.gemm_dequant_nvfp4(ca, sa, Sa, cw, sw, Sw, lora, l2, b)
    assert np.max(np.abs(Y - Yb)) <= 1e-12 * np.max(np.abs(Yb))
    mi, ni = rng.integers(0, M, 20), rng.integers(0, N, 20)
    assert np.array_equal(oracle.gemm_w4a4_nvfp4_at(mi, ni, ca, sa, Sa, cw, sw, Sw, lora, l2, b),
                          Y[mi, ni])


def test_nvfp4_act_stage_definition():
    rng = np.random.default_rng(25)
    M, K = 6, 128
    xb = synth.random_bf16(rng, (M, K), 1.0)
    si = rng.uniform(0.2, 2.0, K).astype(np.float32)
    xhat = synth.bf16_bits_to_f32(xb) * si[None, :]
    S = np.float32(np.max(np.abs(xhat)) / np.float32(2688))
    c, s, _ = oracle.quant_act_nvfp4(xb, si, S)
    # block scales: E4M3 of absmax / (6 S), via torch's cast (no value exceeds 448 here)
    amax = np.abs(xhat).reshape(M, K // 16, 16).max(axis=2)
    sbv = (amax / np.float32(np.float32(6.0) * S)).astype(np.float32)
    ref_s = torch.from_numpy(sbv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(s, ref_s)
    # codes: E2M1 of x / (sb * S)
    d = (oracle.e4m3_decode(s.reshape(-1)).astype(np.float32).reshape(s.shape) * S)
    q = (xhat / np.repeat(d, 16, axis=1)).astype(np.float32)
    ref_c = oracle.e2m1_encode(q.reshape(-1)).reshape(M, K)
    assert np.array_equal(oracle.unpack_u4(c), ref_c)
    # dequantized values are within half a grid step of x
    deq = bf.dequant_nvfp4(c, s, S)
    assert np.all(np.abs(deq - xhat) <= 1.0 * np.repeat(d, 16, axis=1) + 1e-30)

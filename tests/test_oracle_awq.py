"""Pins of the oracle's AWQ W4A16 path (page "Diffusers Natively Integrates Nunchaku Lite
...", third paragraph: modulation layers use 4-bit weights with 16-bit activations).
"""
import numpy as np

import oracle
import synth
from oracle import bruteforce as bf


def _w(rng, N, K):
    return (rng.standard_normal((N, K)) * 0.02).astype(np.float32)


def test_onehot_rows_return_dequantized_columns_plus_bias():
    rng = np.random.default_rng(30)
    N, K = 16, 192
    q, sc, z = oracle.awq_quant_weight(_w(rng, N, K))
    b = synth.random_bf16(rng, (N,), 0.1)
    ks = [0, 1, 63, 64, 130, 191]
    x = np.zeros((len(ks), K), np.float32)
    for i, k in enumerate(ks):
        x[i, k] = 1.0
    Y = oracle.awq_gemv(synth.f32_to_bf16_bits(x), q, sc, z, b)
    deq = bf.dequant_awq(q, sc, z)
    for i, k in enumerate(ks):
        assert np.array_equal(Y[i], deq[:, k] + oracle.bf16_to_f64(b))


def test_on_grid_weights_roundtrip():
    # w = (q - z) * sc with sc a bf16 value, q spanning 0..15 in each group -> exact
    rng = np.random.default_rng(31)
    N, K = 8, 128
    sc = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        np.float32(2.0) ** rng.integers(-8, -3, size=(N, K // 64)).astype(np.float32)))
    z = rng.integers(1, 15, size=(N, K // 64))
    q = rng.integers(0, 16, size=(N, K))
    q[:, ::64], q[:, 1::64] = 0, 15
    w = ((q - np.repeat(z, 64, axis=1)) * np.repeat(sc, 64, axis=1)).astype(np.float32)
    qq, scs, zz = oracle.awq_quant_weight(w)
    assert np.array_equal(oracle.unpack_u4(qq), q.astype(np.uint8))
    assert np.array_equal(synth.bf16_bits_to_f32(scs), sc)
    assert np.array_equal(oracle.bf16_to_f64(zz), z.astype(np.float64))


def test_gemv_equals_dequant_matmul_and_error_bound():
    rng = np.random.default_rng(32)
    M, N, K = 2, 40, 256
    w = _w(rng, N, K)
    q, sc, z = oracle.awq_quant_weight(w)
    x = synth.random_bf16(rng, (M, K), 1.0)
    b = synth.random_bf16(rng, (N,), 0.1)
    Y = oracle.awq_gemv(x, q, sc, z, b)
    deq = bf.dequant_awq(q, sc, z)
    Yb = oracle.bf16_to_f64(x) @ deq.T + oracle.bf16_to_f64(b)[None, :]
    assert np.max(np.abs(Y - Yb)) <= 1e-13
    # quantization error per weight is at most half a step (zero-point rounding can add
    # up to half a step more at the range ends)
    step = np.repeat(oracle.bf16_to_f64(sc), 64, axis=1)
    assert np.all(np.abs(deq - w) <= 1.0 * step + 1e-12)
    # z is an integer in [0, 15] and q in [0, 15]
    zz = oracle.bf16_to_f64(z)
    assert np.all(zz == np.round(zz)) and zz.min() >= 0 and zz.max() <= 15


def test_constant_group_gets_unit_scale():
    N, K = 2, 64
    w = np.full((N, K), 0.5, np.float32)
    q, sc, z = oracle.awq_quant_weight(w)
    assert np.all(sc == 0x3F80)
    deq = bf.dequant_awq(q, sc, z)
    # range 0 -> scale 1, z = clamp(rne(-0.5), 0, 15) = 0, q = rne(0.5) + 0 = 0
    assert np.all(deq == 0.0)

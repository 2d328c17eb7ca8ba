"""Seeded synthetic inputs for the SVDQuant W4A4 linear, its NVFP4 variant and the
AWQ W4A16 GEMV.

This module draws random numbers and nothing else: it holds none of the method's
arithmetic (no smoothing, no factorisation, no quantisation).  It is the only module
that both the HIP path's harness (tests, bench) and the CPU oracle use.

The pages measure end to end on one diffusion transformer at 1024x1024 (ERNIE-Image-
Turbo, RTX PRO 6000; page "Diffusers Natively Integrates Nunchaku Lite ...", third
paragraph).  No dataset or checkpoint is available, so these tensors stand in for a
DiT's activations and weights at that scale:
  * activations: bf16 N(0, 1) with a few outlier channels scaled up after sampling
    (the outliers that make plain W4A4 fail, page "Hugging Face 把 Nunchaku 4-bit
    Diffusion 接到 Diffusers", 技术细节 1);
  * weights: N(0, 0.02^2);  bias: bf16 U(-1/sqrt(K), 1/sqrt(K)) (nn.Linear default);
  * the MLP's second input is heavy tailed (Student-t, 3 degrees of freedom);
  * the AWQ path's per-channel activation magnitudes are LogNormal(0, 1).
Random generator: numpy PCG64 seeded with 42 + workload index; draw order X, outlier
permutation, W, bias, extras.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def f32_to_bf16_bits(a):
    """Round float32 values to bf16 (nearest, ties to even) -> uint16 bit patterns.
    (A dtype conversion of the synthetic inputs, not part of the method.)"""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u                      # wraps only for NaN bit patterns, replaced below
    lsb >>= np.uint32(16)
    out = lsb.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    index: int
    M: int
    K: int
    N: int
    rank: int
    precision: str            # "int4", "nvfp4" or "awq"
    has_bias: bool
    outlier_frac: float
    outlier_scale: float
    # MLP pair only: second linear K2 -> N2 on a Student-t input
    K2: int = 0
    N2: int = 0


WORKLOADS = [
    Workload("tiny_256x512x512_r16", 0, 256, 512, 512, 16, "int4", False, 0.02, 30.0),
    Workload("attn_4096x3072x3072_r32", 1, 4096, 3072, 3072, 32, "int4", True, 0.01, 50.0),
    Workload("mlp_4608x3072x12288x3072_r32", 2, 4608, 3072, 12288, 32, "int4", True, 0.01, 50.0,
             K2=12288, N2=3072),
    Workload("qkv_nvfp4_4096x3072x9216_r32", 3, 4096, 3072, 9216, 32, "nvfp4", True, 0.01, 50.0),
    Workload("awq_gemv_2x3072x18432", 4, 2, 3072, 18432, 0, "awq", True, 0.0, 1.0),
]


def n_outliers(frac, K):
    # round half to even of frac * K (numpy's rint)
    return int(np.rint(frac * K))


@dataclass
class Draws:
    x_bf16: np.ndarray                 # [M, K] uint16
    w: np.ndarray                      # [N, K] float64
    bias_bf16: Optional[np.ndarray]    # [N] uint16 or None
    outlier_channels: np.ndarray
    extras: dict = field(default_factory=dict)


def _activation(rng, M, K, frac, scale, dist="normal"):
    if dist == "normal":
        x = rng.standard_normal((M, K))
    else:
        x = rng.standard_t(3.0, size=(M, K))
    n_out = n_outliers(frac, K)
    ch = np.sort(rng.permutation(K)[:n_out]) if n_out else np.zeros(0, np.int64)
    if n_out:
        x[:, ch] *= scale
    return f32_to_bf16_bits(x.astype(np.float32)), ch


def _bias(rng, N, K):
    b = rng.uniform(-1.0 / np.sqrt(K), 1.0 / np.sqrt(K), size=N)
    return f32_to_bf16_bits(b.astype(np.float32))


def draw(wl: Workload, seed_offset: int = 0, M: Optional[int] = None) -> Draws:
    """Raw random tensors of a workload (optionally with fewer rows M)."""
    rng = np.random.Generator(np.random.PCG64(42 + wl.index + seed_offset))
    M = wl.M if M is None else M
    x, ch = _activation(rng, M, wl.K, wl.outlier_frac, wl.outlier_scale)
    w = rng.normal(0.0, 0.02, size=(wl.N, wl.K))
    bias = _bias(rng, wl.N, wl.K) if wl.has_bias else None
    extras = {}
    if wl.K2:
        x2, ch2 = _activation(rng, M, wl.K2, wl.outlier_frac, wl.outlier_scale, dist="t3")
        extras["x2_bf16"] = x2
        extras["outlier_channels2"] = ch2
        extras["w2"] = rng.normal(0.0, 0.02, size=(wl.N2, wl.K2))
        extras["bias2_bf16"] = _bias(rng, wl.N2, wl.K2)
    if wl.precision == "awq":
        extras["act_magnitude"] = rng.lognormal(0.0, 1.0, size=wl.K)
    return Draws(x, w, bias, ch, extras)


def random_bf16(rng, shape, std):
    return f32_to_bf16_bits((rng.standard_normal(shape) * std).astype(np.float32))


def random_packed_nibbles(rng, rows, K):
    """Uniform random bytes = two random 4-bit codes per byte."""
    return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)

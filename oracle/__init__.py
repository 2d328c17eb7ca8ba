"""CPU oracle for the SVDQuant W4A4 linear, its NVFP4 variant and the AWQ W4A16 GEMV.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with the
HIP library (``bit_diffusion_amd``) and neither imports the other; the only module
both sides use is the seeded input generator ``synth``, which holds no arithmetic
of the method.

Layout:
  svdq_oracle.c   scalar C oracle (fp32 op sequence of the quantizers, exact integer
                  group dots, fp64 accumulation); wrapped here with ctypes.
  bruteforce.py   independent NumPy fp64 formulations used to pin the C oracle.
  construct.py    offline weight construction (smoothing factors, top-r factors,
                  residual quantization; AWQ weights) in NumPy fp64 + the C quantizers.

bf16 tensors are passed as uint16 bit patterns, fp8/fp4/int4 codes as uint8.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """Load (building if needed) oracle/liboracle.so."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        sig = {
            "oracle_f64_to_bf16": ([ctypes.c_double], ctypes.c_uint16),
            "oracle_f32_to_bf16": ([F], ctypes.c_uint16),
            "oracle_e4m3_decode": ([ctypes.c_uint8], ctypes.c_double),
            "oracle_e4m3_encode": ([F], ctypes.c_uint8),
            "oracle_e2m1_decode": ([ctypes.c_uint8], ctypes.c_double),
            "oracle_e2m1_encode": ([F], ctypes.c_uint8),
            "oracle_quant_act_int4": ([I64, I64, I, P, P, P, P, P, P], None),
            "oracle_quant_rows_int4": ([I64, I64, P, P, P], None),
            "oracle_gemm_w4a4_int4": ([I64, I64, I64, I, P, P, P, P, P, P, P, I, P], None),
            "oracle_gemm_w4a4_int4_at": ([I64, P, P, I64, I, P, P, P, P, P, P, P, I, P], None),
            "oracle_quant_act_nvfp4": ([I64, I64, I, P, P, P, F, P, P, P], None),
            "oracle_quant_rows_nvfp4": ([I64, I64, P, F, P, P], None),
            "oracle_gemm_w4a4_nvfp4": ([I64, I64, I64, I, P, P, F, P, P, F, P, P, P, I, P], None),
            "oracle_gemm_w4a4_nvfp4_at": ([I64, P, P, I64, I, P, P, F, P, P, F, P, P, P, I, P],
                                          None),
            "oracle_awq_quant_weight": ([I64, I64, P, P, P, P], None),
            "oracle_awq_gemv": ([I64, I64, I64, P, P, P, P, P, P], None),
            "oracle_gelu_tanh": ([I64, P, P], None),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


# ------------------------------------------------------------------ scalar helpers

def bf16_from_f64(d):
    """Nearest bf16 (one rounding, ties to even) of binary64 values -> uint16."""
    L = lib()
    d = np.asarray(d, dtype=np.float64)
    out = np.empty(d.shape, dtype=np.uint16)
    flat, of = d.reshape(-1), out.reshape(-1)
    for i in range(flat.size):
        of[i] = L.oracle_f64_to_bf16(float(flat[i]))
    return out


def bf16_to_f64(h):
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_encode(v):
    L = lib()
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    return np.array([L.oracle_e4m3_encode(float(x)) for x in v], dtype=np.uint8)


def e4m3_decode(b):
    L = lib()
    b = np.asarray(b, dtype=np.uint8).reshape(-1)
    return np.array([L.oracle_e4m3_decode(int(x)) for x in b], dtype=np.float64)


def e2m1_encode(v):
    L = lib()
    v = np.asarray(v, dtype=np.float32).reshape(-1)
    return np.array([L.oracle_e2m1_encode(float(x)) for x in v], dtype=np.uint8)


def e2m1_decode(c):
    L = lib()
    c = np.asarray(c, dtype=np.uint8).reshape(-1)
    return np.array([L.oracle_e2m1_decode(int(x)) for x in c], dtype=np.float64)


# ------------------------------------------------------------------ INT4

def quant_act_int4(x_bf16, smooth_inv, l1_bf16=None):
    """Activation stage (INT4): returns codes [M,K/2] u8, scales [M,K/64] f32,
    lora [M,r] bf16 (uint16; shape [M,0] when r == 0)."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    si = _c(smooth_inv, np.float32)
    r = 0 if l1_bf16 is None else l1_bf16.shape[0]
    l1 = _c(l1_bf16, np.uint16) if r else None
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 64), np.float32)
    lora = np.empty((M, r), np.uint16)
    lib().oracle_quant_act_int4(M, K, r, _p(x), _p(si), _p(l1), _p(codes), _p(scales),
                                _p(lora))
    return codes, scales, lora


def quant_rows_int4(vals_f32):
    v = _c(vals_f32, np.float32)
    R, K = v.shape
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 64), np.float32)
    lib().oracle_quant_rows_int4(R, K, _p(v), _p(codes), _p(scales))
    return codes, scales


def gemm_w4a4_int4(ca, sa, cw, sw, lora=None, l2=None, bias=None, act=0):
    ca, sa = _c(ca, np.uint8), _c(sa, np.float32)
    cw, sw = _c(cw, np.uint8), _c(sw, np.float32)
    M, K = ca.shape[0], ca.shape[1] * 2
    N = cw.shape[0]
    r = 0 if (lora is None or l2 is None) else lora.shape[1]
    lora = _c(lora, np.uint16) if r else None
    l2 = _c(l2, np.uint16) if r else None
    bias = _c(bias, np.uint16)
    out = np.empty((M, N), np.float64)
    lib().oracle_gemm_w4a4_int4(M, N, K, r, _p(ca), _p(sa), _p(cw), _p(sw), _p(lora), _p(l2),
                                _p(bias), act, _p(out))
    return out


def gemm_w4a4_int4_at(mi, ni, ca, sa, cw, sw, lora=None, l2=None, bias=None, act=0):
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    ca, sa = _c(ca, np.uint8), _c(sa, np.float32)
    cw, sw = _c(cw, np.uint8), _c(sw, np.float32)
    K = ca.shape[1] * 2
    r = 0 if (lora is None or l2 is None) else lora.shape[1]
    lora = _c(lora, np.uint16) if r else None
    l2 = _c(l2, np.uint16) if r else None
    bias = _c(bias, np.uint16)
    out = np.empty(mi.shape[0], np.float64)
    lib().oracle_gemm_w4a4_int4_at(mi.shape[0], _p(mi), _p(ni), K, r, _p(ca), _p(sa), _p(cw),
                                   _p(sw), _p(lora), _p(l2), _p(bias), act, _p(out))
    return out


def merge_lora(l1, l2, lora_down, lora_up, alpha):
    """A LoRA adapter y += alpha (x A^T) B^T merged into the low-rank branch (page "Diffusers
    integra Nunchaku ...", "Nunchaku Lite: integración y modelo de ejecución": LoRA keeps
    working with the SVDQ modules).  The branch computes lora_act = x l1^T and adds
    lora_act l2^T, so the adapter is appended to its factors: l1' = [l1; A; 0],
    l2' = [l2 | bf16(alpha B) | 0], the rank padded with zeros to a multiple of 16.  alpha B
    is one fp32 product per element, rounded to nearest-even bf16.  l1 [r, K], l2 [N, r] (or
    None for r = 0), A [rl, K], B [N, rl]: bf16 bit patterns."""
    down = _c(lora_down, np.uint16)
    up = _c(lora_up, np.uint16)
    rl, K = down.shape
    N = up.shape[0]
    r = 0 if l1 is None else l1.shape[0]
    ro = (r + rl + 15) // 16 * 16
    l1o = np.zeros((ro, K), np.uint16)
    l2o = np.zeros((N, ro), np.uint16)
    if r:
        l1o[:r] = l1
        l2o[:, :r] = l2
    l1o[r:r + rl] = down
    prod = np.float32(alpha) * bf16_to_f64(up).astype(np.float32)   # fp32 product
    l2o[:, r:r + rl] = bf16_from_f64(prod.astype(np.float64))
    return l1o, l2o


# ------------------------------------------------------------------ NVFP4

def quant_act_nvfp4(x_bf16, smooth_inv, S, l1_bf16=None):
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    si = _c(smooth_inv, np.float32)
    r = 0 if l1_bf16 is None else l1_bf16.shape[0]
    l1 = _c(l1_bf16, np.uint16) if r else None
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 16), np.uint8)
    lora = np.empty((M, r), np.uint16)
    lib().oracle_quant_act_nvfp4(M, K, r, _p(x), _p(si), _p(l1), float(np.float32(S)),
                                 _p(codes), _p(scales), _p(lora))
    return codes, scales, lora


def quant_rows_nvfp4(vals_f32, S):
    v = _c(vals_f32, np.float32)
    R, K = v.shape
    codes = np.empty((R, K // 2), np.uint8)
    scales = np.empty((R, K // 16), np.uint8)
    lib().oracle_quant_rows_nvfp4(R, K, _p(v), float(np.float32(S)), _p(codes), _p(scales))
    return codes, scales


def gemm_w4a4_nvfp4(ca, sa, Sa, cw, sw, Sw, lora=None, l2=None, bias=None, act=0):
    ca, sa = _c(ca, np.uint8), _c(sa, np.uint8)
    cw, sw = _c(cw, np.uint8), _c(sw, np.uint8)
    M, K = ca.shape[0], ca.shape[1] * 2
    N = cw.shape[0]
    r = 0 if (lora is None or l2 is None) else lora.shape[1]
    lora = _c(lora, np.uint16) if r else None
    l2 = _c(l2, np.uint16) if r else None
    bias = _c(bias, np.uint16)
    out = np.empty((M, N), np.float64)
    lib().oracle_gemm_w4a4_nvfp4(M, N, K, r, _p(ca), _p(sa), float(np.float32(Sa)), _p(cw),
                                 _p(sw), float(np.float32(Sw)), _p(lora), _p(l2), _p(bias),
                                 act, _p(out))
    return out


def gemm_w4a4_nvfp4_at(mi, ni, ca, sa, Sa, cw, sw, Sw, lora=None, l2=None, bias=None, act=0):
    mi = _c(np.asarray(mi, np.int64), np.int64)
    ni = _c(np.asarray(ni, np.int64), np.int64)
    ca, sa = _c(ca, np.uint8), _c(sa, np.uint8)
    cw, sw = _c(cw, np.uint8), _c(sw, np.uint8)
    K = ca.shape[1] * 2
    r = 0 if (lora is None or l2 is None) else lora.shape[1]
    lora = _c(lora, np.uint16) if r else None
    l2 = _c(l2, np.uint16) if r else None
    bias = _c(bias, np.uint16)
    out = np.empty(mi.shape[0], np.float64)
    lib().oracle_gemm_w4a4_nvfp4_at(mi.shape[0], _p(mi), _p(ni), K, r, _p(ca), _p(sa),
                                    float(np.float32(Sa)), _p(cw), _p(sw),
                                    float(np.float32(Sw)), _p(lora), _p(l2), _p(bias), act,
                                    _p(out))
    return out


# ------------------------------------------------------------------ AWQ

def awq_quant_weight(w_f32):
    w = _c(w_f32, np.float32)
    N, K = w.shape
    q = np.empty((N, K // 2), np.uint8)
    sc = np.empty((N, K // 64), np.uint16)
    z = np.empty((N, K // 64), np.uint16)
    lib().oracle_awq_quant_weight(N, K, _p(w), _p(q), _p(sc), _p(z))
    return q, sc, z


def awq_gemv(x_bf16, q, sc, z, bias=None):
    x = _c(x_bf16, np.uint16)
    q, sc, z = _c(q, np.uint8), _c(sc, np.uint16), _c(z, np.uint16)
    bias = _c(bias, np.uint16)
    M, K = x.shape
    N = q.shape[0]
    out = np.empty((M, N), np.float64)
    lib().oracle_awq_gemv(M, N, K, _p(x), _p(q), _p(sc), _p(z), _p(bias), _p(out))
    return out


def gelu_tanh(y):
    y = _c(np.asarray(y, np.float64), np.float64)
    out = np.empty_like(y)
    lib().oracle_gelu_tanh(y.size, _p(y), _p(out))
    return out


# ------------------------------------------------------------------ code unpacking

def unpack_int4(codes):
    """[R, K/2] two's-complement nibbles (low nibble = even k) -> int8 [R, K]."""
    c = np.asarray(codes, np.uint8)
    lo = (c & 0x0F).astype(np.int16)
    hi = (c >> 4).astype(np.int16)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.int16)
    out[:, 0::2], out[:, 1::2] = lo, hi
    out = np.where(out >= 8, out - 16, out)
    return out.astype(np.int8)


def unpack_u4(codes):
    """[R, K/2] unsigned nibbles (low nibble = even k) -> uint8 [R, K]."""
    c = np.asarray(codes, np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2], out[:, 1::2] = c & 0x0F, c >> 4
    return out

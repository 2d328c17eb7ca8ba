"""Helpers for GPU tests: numpy <-> device tensors and calls through the C ABI."""
import numpy as np
import torch

import bit_diffusion_amd as bd


def dev(a):
    """numpy -> torch tensor on cuda:0 with the same bytes (bf16 words travel as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to("cuda:0")


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if t.dtype == torch.int16:
        a = a.view(np.uint16)
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty(shape, dtype):
    tmap = {np.uint8: torch.uint8, np.uint16: torch.int16, np.float32: torch.float32}
    return torch.empty(shape, dtype=tmap[dtype], device="cuda:0")


def quantize(x_bf16, smooth_inv, l1=None, precision="int4", S=1.0, N=1):
    """Run svdq_quantize_act on device inputs (numpy or tensors) -> (codes, scales, lora) tensors."""
    x = x_bf16 if torch.is_tensor(x_bf16) else dev(x_bf16)
    M, K = x.shape
    r = 0 if l1 is None else l1.shape[0]
    cfg = bd.LayerCfg.make(K, N, r, precision)
    codes = empty((M, K // 2), np.uint8)
    scales = empty((M, K // 64), np.float32) if precision == "int4" else empty((M, K // 16), np.uint8)
    lora = empty((M, r), np.uint16) if r else None
    si = smooth_inv if torch.is_tensor(smooth_inv) else dev(np.asarray(smooth_inv, np.float32))
    l1d = None if l1 is None else (l1 if torch.is_tensor(l1) else dev(l1))
    bd.svdq_quantize_act(cfg, M, x, si, l1d, S, codes, scales, lora)
    return codes, scales, lora


def gemm(codes, scales, wcodes, wscales, lora=None, l2=None, bias=None, act=0, out_bf16=False,
         precision="int4", Sa=1.0, Sw=1.0):
    M = codes.shape[0]
    K = codes.shape[1] * 2
    wc = wcodes if torch.is_tensor(wcodes) else dev(wcodes)
    ws = wscales if torch.is_tensor(wscales) else dev(wscales)
    N = wc.shape[0]
    r = 0 if lora is None else lora.shape[1]
    l2d = None if l2 is None or r == 0 else (l2 if torch.is_tensor(l2) else dev(l2))
    bd_ = None if bias is None else (bias if torch.is_tensor(bias) else dev(bias))
    lo = None if r == 0 else (lora if torch.is_tensor(lora) else dev(lora))
    cfg = bd.LayerCfg.make(K, N, r, precision)
    out = empty((M, N), np.uint16 if out_bf16 else np.float32)
    c = codes if torch.is_tensor(codes) else dev(codes)
    s = scales if torch.is_tensor(scales) else dev(scales)
    bd.svdq_gemm_w4a4(cfg, M, c, s, Sa, wc, ws, Sw, lo, l2d, bd_, act,
                      bd.SVDQ_DT_BF16 if out_bf16 else bd.SVDQ_DT_F32, out)
    return out


def prepack(wcodes, wscales, K, N):
    cfg = bd.LayerCfg.make(K, N, 0)
    nbytes = bd.svdq_prepacked_weight_bytes(cfg)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    wc = wcodes if torch.is_tensor(wcodes) else dev(wcodes)
    ws = wscales if torch.is_tensor(wscales) else dev(wscales)
    bd.svdq_prepack_weight(cfg, wc, ws, buf)
    return buf


def act_packed_bytes(M, K):
    return bd.svdq_act_packed_bytes(bd.LayerCfg.make(K, 1, 0), M)


def pack_act(codes, scales, K):
    """svdq_pack_act: nibble codes + fp32 scales -> packed activation buffer."""
    c = codes if torch.is_tensor(codes) else dev(codes)
    s = scales if torch.is_tensor(scales) else dev(scales)
    M = c.shape[0]
    buf = torch.empty(act_packed_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    bd.svdq_pack_act(bd.LayerCfg.make(K, 1, 0), M, c, s, buf)
    return buf


def quantize_packed(x_bf16, smooth_inv, l1=None, N=1, with_scales=True):
    """svdq_quantize_act_packed -> (packed buffer, fp32 scales or None, lora) tensors."""
    x = x_bf16 if torch.is_tensor(x_bf16) else dev(x_bf16)
    M, K = x.shape
    r = 0 if l1 is None else l1.shape[0]
    cfg = bd.LayerCfg.make(K, N, r)
    buf = torch.empty(act_packed_bytes(M, K), dtype=torch.uint8, device="cuda:0")
    scales = empty((M, K // 64), np.float32) if with_scales else None
    lora = empty((M, r), np.uint16) if r else None
    si = smooth_inv if torch.is_tensor(smooth_inv) else dev(np.asarray(smooth_inv, np.float32))
    l1p = None if l1 is None else prepack_l1(l1, K)
    bd.svdq_quantize_act_packed(cfg, M, x, si, l1p, buf, scales, lora)
    return buf, scales, lora


def prepack_l1(l1, K):
    """svdq_prepack_l1: bf16 bits [r, K] -> the prepacked low-rank factor."""
    l1d = l1 if torch.is_tensor(l1) else dev(l1)
    cfg = bd.LayerCfg.make(K, 1, l1d.shape[0])
    out = torch.empty(bd.svdq_prepacked_l1_bytes(cfg), dtype=torch.uint8, device="cuda:0")
    bd.svdq_prepack_l1(cfg, l1d, out)
    return out


def gemm_packed(apacked, wpacked, M, K, N, lora=None, l2=None, bias=None, act=0, out_bf16=False):
    r = 0 if lora is None else lora.shape[1]
    l2d = None if l2 is None or r == 0 else (l2 if torch.is_tensor(l2) else dev(l2))
    bd_ = None if bias is None else (bias if torch.is_tensor(bias) else dev(bias))
    lo = None if r == 0 else (lora if torch.is_tensor(lora) else dev(lora))
    cfg = bd.LayerCfg.make(K, N, r)
    out = empty((M, N), np.uint16 if out_bf16 else np.float32)
    bd.svdq_gemm_w4a4_packed(cfg, M, apacked, wpacked, lo, l2d, bd_, act,
                             bd.SVDQ_DT_BF16 if out_bf16 else bd.SVDQ_DT_F32, out)
    return out


def gemm_prepacked(codes, scales, packed, N, lora=None, l2=None, bias=None, act=0,
                   out_bf16=False):
    """Nibble activations -> svdq_pack_act -> svdq_gemm_w4a4_packed."""
    M = codes.shape[0]
    K = codes.shape[1] * 2
    return gemm_packed(pack_act(codes, scales, K), packed, M, K, N, lora, l2, bias, act,
                       out_bf16)


def _fp6_fields(dw):
    """[..., 6] uint32 dwords -> [..., 32] six-bit fields (field j at bit 6 j)."""
    dw = dw.astype(np.uint64)
    out = np.empty(dw.shape[:-1] + (32,), np.int64)
    for j in range(32):
        pos = 6 * j
        d, o = pos // 32, pos % 32
        f = dw[..., d] >> np.uint64(o)
        if o > 26:
            f = f | (dw[..., d + 1] << np.uint64(32 - o))
        out[..., j] = (f & np.uint64(63)).astype(np.int64)
    return out


def decode_act_packed(buf, M, K):
    """Host-side reader of the packed activation layout (test infrastructure): returns the
    int codes [Mp, K], the scale pairs (h | m << 16, l) [Mp, G, 2] and a flag that every
    field is canonical (no negative zero, magnitude <= 8)."""
    G = K // 64
    mb = (M + 255) // 256
    b = np.ascontiguousarray(np.asarray(buf, np.uint8)).reshape(mb, G, 8, 1792)
    p0 = np.ascontiguousarray(b[..., :1024]).view(np.uint32).reshape(mb, G, 8, 64, 4)
    p1 = np.ascontiguousarray(b[..., 1024:1536]).view(np.uint32).reshape(mb, G, 8, 64, 2)
    f = _fp6_fields(np.concatenate([p0, p1], axis=-1))          # mb, G, rb, lane, j
    mag, neg = f & 31, f >> 5
    canonical = bool(np.all(mag <= 8) and not np.any((mag == 0) & (neg == 1)))
    q = np.where(neg == 1, -mag, mag).reshape(mb, G, 8, 2, 32, 32)  # lane = r + 32 h
    codes = q.transpose(0, 2, 4, 1, 3, 5).reshape(mb * 256, K)
    words = np.ascontiguousarray(b[..., 1536:]).view(np.uint32).reshape(mb, G, 8, 32, 2)
    words = words.transpose(0, 2, 3, 1, 4).reshape(mb * 256, G, 2)
    return codes, words, canonical


def split_words(scales):
    """The scale pair the packed layout stores per (row, group): (h | m << 16, l) with
    h = bf16(s), m = bf16(s - h), l = bf16(s - h - m)."""
    import synth
    s = np.asarray(scales, np.float32)
    h = synth.f32_to_bf16_bits(s).astype(np.uint32)
    r1 = (s - (h << 16).view(np.float32)).astype(np.float32)
    m = synth.f32_to_bf16_bits(r1).astype(np.uint32)
    r2 = (r1 - (m << 16).view(np.float32)).astype(np.float32)
    l = synth.f32_to_bf16_bits(r2).astype(np.uint32)
    return np.stack([h | (m << 16), l], axis=-1)


def awq(x_bf16, q, sc, z, bias=None, out_bf16=False):
    x = x_bf16 if torch.is_tensor(x_bf16) else dev(x_bf16)
    M, K = x.shape
    qd = q if torch.is_tensor(q) else dev(q)
    N = qd.shape[0]
    out = empty((M, N), np.uint16 if out_bf16 else np.float32)
    bd.awq_gemm_w4a16(M, K, N, 64, x, qd, dev(sc), dev(z), None if bias is None else dev(bias),
                      bd.SVDQ_DT_BF16 if out_bf16 else bd.SVDQ_DT_F32, out)
    return out


def rel_fro(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_ulp_diff(a, b):
    """Distance in bf16 ulps between two arrays of bf16 bit patterns (same sign assumed
    where both are nonzero)."""
    a = np.asarray(a, np.uint16).astype(np.int32)
    b = np.asarray(b, np.uint16).astype(np.int32)
    # map to a monotone integer line
    ia = np.where(a & 0x8000, -(a & 0x7FFF), a)
    ib = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ia - ib)


def assert_bf16_close(bits, ref, min_exact=0.99):
    """bf16 results vs an fp64 reference: each element within one bf16 ulp of the reference
    plus an absolute slack of 2^-16 of the largest |reference| (fp32 accumulation error on
    elements that cancel to near zero, which GELU's negative tail also magnifies), and at
    least `min_exact` of the elements above 1% of the largest magnitude bit-equal to the
    reference rounded to bf16."""
    from oracle.construct import bf16_from_f64_vec
    ref = np.asarray(ref, np.float64)
    got = (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = np.abs(ref)
    _, e = np.frexp(np.maximum(a, 1e-38))
    ulp = np.ldexp(1.0, e - 8)
    tol = ulp + np.ldexp(np.max(a), -16)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (f"{bad.sum()} bf16 elements off: worst "
                           f"{np.max(np.abs(got - ref)[bad])} vs tol {tol[bad][0]}")
    # exactness is expected where the fp32 accumulation error (~1e-7 of the largest terms)
    # is far below a bf16 ulp: elements at least 1% of the largest magnitude
    big = a >= 1e-2 * np.max(a)
    exact = np.mean(np.asarray(bits, np.uint16)[big] == bf16_from_f64_vec(ref[big]))
    assert exact >= min_exact, f"only {exact:.4f} of bf16 outputs exact"


def assert_lora_close(got_bits, oracle_bits, x_bf16, l1_bf16, min_exact=0.99):
    """lora_act from the GPU (fp32 accumulation, one bf16 rounding) vs the oracle (fp64 sum,
    one bf16 rounding): within one bf16 ulp of the exact sum plus the fp32 summation error
    bound 2^-16 * sum_k |x_k l1_jk|, and at least `min_exact` bit-equal to the oracle."""
    from oracle import bf16_to_f64
    x = bf16_to_f64(x_bf16)
    l1 = bf16_to_f64(l1_bf16)
    exact = x @ l1.T
    cond = np.abs(x) @ np.abs(l1).T
    got = bf16_to_f64(got_bits)
    _, e = np.frexp(np.maximum(np.abs(exact), 1e-38))
    tol = np.ldexp(1.0, e - 8) + np.ldexp(cond, -16)
    bad = np.abs(got - exact) > tol
    assert not bad.any(), f"{bad.sum()} lora_act elements beyond the fp32 error bound"
    frac = np.mean(np.asarray(got_bits) == np.asarray(oracle_bits))
    assert frac >= min_exact, f"only {frac:.4f} of lora_act equal to the oracle"


def gemm_packed_quantize_next(apacked, wpacked, M, K, N, lora, l2, bias, act, next_si, next_l1,
                              with_scales=True):
    """svdq_gemm_w4a4_packed_quantize_next: the packed GEMM with the next layer's activation
    kernel in its epilogue -> (next packed buffer, fp32 scales or None, next lora_act)."""
    r = 0 if lora is None else lora.shape[1]
    r2 = 0 if next_l1 is None else next_l1.shape[0]
    cfg = bd.LayerCfg.make(K, N, r)
    ncfg = bd.LayerCfg.make(N, 1, r2)
    l2d = None if l2 is None or r == 0 else (l2 if torch.is_tensor(l2) else dev(l2))
    bd_ = None if bias is None else (bias if torch.is_tensor(bias) else dev(bias))
    lo = None if r == 0 else (lora if torch.is_tensor(lora) else dev(lora))
    si = next_si if torch.is_tensor(next_si) else dev(np.asarray(next_si, np.float32))
    l1d = None if r2 == 0 else (next_l1 if torch.is_tensor(next_l1) else dev(next_l1))
    buf = torch.empty(act_packed_bytes(M, N), dtype=torch.uint8, device="cuda:0")
    scales = empty((M, N // 64), np.float32) if with_scales else None
    nlora = empty((M, r2), np.uint16) if r2 else None
    work = empty((M, r2), np.float32) if r2 else None
    bd.svdq_gemm_w4a4_packed_quantize_next(cfg, M, apacked, wpacked, lo, l2d, bd_, act, ncfg, si,
                                           l1d, buf, scales, nlora, work)
    return buf, scales, nlora

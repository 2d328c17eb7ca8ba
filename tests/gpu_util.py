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


def gemm_packed(apacked, wpacked, M, K, N, lora=None, l2=None, bias=None, act=0, out_bf16=False,
                split=False):
    """svdq_gemm_w4a4_packed, or with split=True svdq_gemm_w4a4_packed_ws with the workspace
    the library asks for (K split of a nearly empty last round of tiles)."""
    r = 0 if lora is None else lora.shape[1]
    l2d = None if l2 is None or r == 0 else (l2 if torch.is_tensor(l2) else dev(l2))
    bd_ = None if bias is None else (bias if torch.is_tensor(bias) else dev(bias))
    lo = None if r == 0 else (lora if torch.is_tensor(lora) else dev(lora))
    cfg = bd.LayerCfg.make(K, N, r)
    out = empty((M, N), np.uint16 if out_bf16 else np.float32)
    dt = bd.SVDQ_DT_BF16 if out_bf16 else bd.SVDQ_DT_F32
    if split:
        nb = bd.svdq_gemm_w4a4_packed_workspace_bytes(cfg, M, act, dt)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda:0")
        bd.svdq_gemm_w4a4_packed_ws(cfg, M, apacked, wpacked, lo, l2d, bd_, act, dt, out, ws, nb)
    else:
        bd.svdq_gemm_w4a4_packed(cfg, M, apacked, wpacked, lo, l2d, bd_, act, dt, out)
    return out


def split_workspace_bytes(M, K, N, act=0, out_bf16=False):
    return bd.svdq_gemm_w4a4_packed_workspace_bytes(
        bd.LayerCfg.make(K, N, 0), M, act, bd.SVDQ_DT_BF16 if out_bf16 else bd.SVDQ_DT_F32)


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
    int codes [Mp, K], the scale pairs (h | h << 16, m | l << 16) [Mp, G, 2] and a flag that every
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
    """The scale pair the packed layout stores per (row, group): (h | h << 16, m | l << 16)
    with h = bf16(s), m = bf16(s - h), l = bf16(s - h - m)."""
    import synth
    s = np.asarray(scales, np.float32)
    h = synth.f32_to_bf16_bits(s).astype(np.uint32)
    r1 = (s - (h << 16).view(np.float32)).astype(np.float32)
    m = synth.f32_to_bf16_bits(r1).astype(np.uint32)
    r2 = (r1 - (m << 16).view(np.float32)).astype(np.float32)
    l = synth.f32_to_bf16_bits(r2).astype(np.uint32)
    return np.stack([h | (h << 16), m | (l << 16)], axis=-1)


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


U32 = 2.0 ** -24   # unit roundoff of fp32


def int4_nround(K, r):
    """Rounding budget (in units of 2^-24 of the condition sum) of the INT4 GEMMs' fp32
    arithmetic, twice the count below for safety.  Per 64-channel group one rounding of the
    running sum (fma or add), plus the product errors, which add up to at most 8 units of
    the condition sum in total (nibble-operand kernel: scale product and product, 2 units;
    packed kernel: the eight-term scale-product MFMA, 7 units, and the three-term bf16
    splits with the two cross terms the MFMA's operands leave out, under 2^-1); r for the
    low-rank MFMA's sums; the bias, and the K split's fixed-order sum of up to 8 parts."""
    return 2 * (K // 64 + r + 8 + 1 + 8)


def int4_cond(ca, sa, cw, sw, lora=None, l2=None, bias=None, mi=None, ni=None, chunk=256):
    """Condition sum of each INT4 GEMM output at the points (mi[i], ni[i]) (every point when
    both are None): sum_g sa sw sum_k |qa qw| + sum_j |lora l2| + |b|, in fp64.  Every
    partial sum the fp32 arithmetic forms is bounded by it."""
    from oracle import unpack_int4, bf16_to_f64
    ca, cw = np.asarray(ca), np.asarray(cw)
    if mi is None:
        mi, ni = np.meshgrid(np.arange(ca.shape[0]), np.arange(cw.shape[0]), indexing="ij")
        shape = mi.shape
        mi, ni = mi.reshape(-1), ni.reshape(-1)
    else:
        shape = np.shape(mi)
        mi, ni = np.asarray(mi).reshape(-1), np.asarray(ni).reshape(-1)
    K = ca.shape[1] * 2
    G = K // 64
    out = np.empty(mi.shape[0], np.float64)
    for a in range(0, mi.shape[0], chunk):
        m, n = mi[a:a + chunk], ni[a:a + chunk]
        qa = np.abs(unpack_int4(ca[m]).astype(np.float64))
        qw = np.abs(unpack_int4(cw[n]).astype(np.float64))
        d = (qa * qw).reshape(-1, G, 64).sum(-1)
        c = (d * np.asarray(sa, np.float64)[m] * np.asarray(sw, np.float64)[n]).sum(-1)
        if lora is not None and np.shape(lora)[1] > 0:
            c += (np.abs(bf16_to_f64(np.asarray(lora)[m])) * np.abs(bf16_to_f64(np.asarray(l2)[n]))).sum(-1)
        if bias is not None:
            c += np.abs(bf16_to_f64(np.asarray(bias)[n]))
        out[a:a + chunk] = c
    return out.reshape(shape)


def _points(nrows, ncols, mi, ni):
    if mi is None:
        mi, ni = np.meshgrid(np.arange(nrows), np.arange(ncols), indexing="ij")
    shape = np.shape(mi)
    return np.asarray(mi).reshape(-1), np.asarray(ni).reshape(-1), shape


def nvfp4_nround(K, r):
    """Rounding budget of the NVFP4 GEMMs (exact E2M1 x E4M3 products, fp32 sums over K in
    any order, the per-tensor scale products, the low-rank sums, the bias), doubled."""
    return 2 * (K + r + 8)


def nvfp4_cond(ca, sba, Sa, cw, sbw, Sw, lora=None, l2=None, bias=None, mi=None, ni=None,
               chunk=128):
    """Condition sum of each NVFP4 GEMM output: Sa Sw sum_k |ea sba ew sbw| + sum_j |lora l2|
    + |b| (fp64)."""
    from oracle import unpack_u4, e2m1_decode, e4m3_decode, bf16_to_f64
    ca, cw = np.asarray(ca), np.asarray(cw)
    mi, ni, shape = _points(ca.shape[0], cw.shape[0], mi, ni)
    K = ca.shape[1] * 2
    tab = np.abs(e2m1_decode(np.arange(16, dtype=np.uint8)))
    s8 = np.abs(e4m3_decode(np.arange(256, dtype=np.uint8)))
    out = np.empty(mi.shape[0], np.float64)
    for a in range(0, mi.shape[0], chunk):
        m, n = mi[a:a + chunk], ni[a:a + chunk]
        va = tab[unpack_u4(ca[m])] * np.repeat(s8[np.asarray(sba)[m]], 16, axis=1)
        vw = tab[unpack_u4(cw[n])] * np.repeat(s8[np.asarray(sbw)[n]], 16, axis=1)
        c = (va * vw).sum(-1) * float(Sa) * float(Sw)
        if lora is not None and np.shape(lora)[1] > 0:
            c += (np.abs(bf16_to_f64(np.asarray(lora)[m])) * np.abs(bf16_to_f64(np.asarray(l2)[n]))).sum(-1)
        if bias is not None:
            c += np.abs(bf16_to_f64(np.asarray(bias)[n]))
        out[a:a + chunk] = c
    assert K == va.shape[1]
    return out.reshape(shape)


def awq_nround(K):
    """Rounding budget of the AWQ GEMV (fp32 sums of x (128 + q) over each group, the zero
    point term, the scale products and the sum over groups, the bias), doubled."""
    return 2 * (K + 2 * (K // 64) + 8)


# The AWQ GEMV sums x (128 + q) and subtracts (128 + z) sum x per group: its fp32 partial
# sums are ~16x the result's terms, so more of its bf16 outputs sit within the fp32 error
# of a rounding boundary than the INT4 GEMMs' (measured 99.5-99.9 % bit-equal).
AWQ_MIN_EXACT = 0.99


def awq_cond(x_bf16, q, sc, z, bias=None):
    """Condition sum of each AWQ output [M, N]: sum_g s_g (sum_k |x_k| (128 + q_k) + (128 + z_g)
    sum_k |x_k|) + |b|, the magnitude bound of every partial sum of the bf16-MFMA form
    (codes taken as 128 + q, the zero point as (128 + z) sum x)."""
    from oracle import unpack_u4, bf16_to_f64
    x = np.abs(bf16_to_f64(x_bf16))
    qv = unpack_u4(np.asarray(q)).astype(np.float64) + 128.0     # [N, K]
    s = np.abs(bf16_to_f64(sc))                                   # [N, G]
    zz = bf16_to_f64(z) + 128.0
    M, K = x.shape
    G = K // 64
    xs = x.reshape(M, G, 64).sum(-1)                              # [M, G]
    t1 = np.einsum("mgk,ngk->mng", x.reshape(M, G, 64), qv.reshape(-1, G, 64))
    c = ((t1 + xs[:, None, :] * zz[None, :, :]) * s[None, :, :]).sum(-1)
    if bias is not None:
        c += np.abs(bf16_to_f64(bias))[None, :]
    return c


def bound_of(cond, nround, gelu=False):
    """Absolute error bound of an fp32 result with condition sum `cond` and `nround`
    roundings; through GELU(tanh) (slope <= 1.13, fp32 evaluation within 32 roundings of the
    argument's magnitude) when gelu."""
    e = nround * U32 * np.asarray(cond, np.float64)
    if gelu:
        e = 1.2 * e + 32 * U32 * np.asarray(cond, np.float64)
    return e


def assert_f32_within(y, ref, cond, nround, gelu=False):
    """fp32 outputs: |y - ref| <= the fp32 error bound, element by element."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    e = bound_of(cond, nround, gelu)
    err = np.abs(y - ref)
    bad = err > e
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} fp32 outputs beyond the fp32 error "
                           f"bound: worst excess {np.max(err[bad] / e[bad]):.2f}x")
    return float(np.max(err / np.maximum(e, 1e-300)))


def _bf16_val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_bf16_close(bits, ref, cond=None, nround=None, gelu=False, min_exact=None):
    """bf16 results vs an fp64 reference.  With the condition sums `cond` and the rounding
    budget `nround` of the fp32 arithmetic: every element is one of the bf16 values that
    round-to-nearest-even of some fp32 value within the error bound of `ref` gives, i.e. lies
    in [bf16(ref - e), bf16(ref + e)] (so it is bit-equal to bf16(ref) wherever that interval
    holds no rounding boundary).  Without them: within one bf16 ulp of ref plus 2^-16 of the
    largest |ref|.  In both cases at least `min_exact` of all elements are bit-equal to
    bf16(ref): 0.998 by default, 0.9 after GELU, whose negative tail gives outputs near zero
    next to their condition sums (fp32 rounding there spans several bf16 values).  Returns
    the bit-equal fraction."""
    if min_exact is None:
        min_exact = 0.9 if gelu else 0.998
    from oracle.construct import bf16_from_f64_vec
    ref = np.asarray(ref, np.float64)
    bits = np.asarray(bits, np.uint16)
    got = _bf16_val(bits)
    if cond is not None:
        e = bound_of(cond, nround, gelu)
        lo = _bf16_val(bf16_from_f64_vec(ref - e))
        hi = _bf16_val(bf16_from_f64_vec(ref + e))
        bad = (got < lo) | (got > hi)
        assert not bad.any(), (f"{int(bad.sum())} of {bad.size} bf16 outputs outside the rounding "
                               f"range of the fp32 error bound")
    else:
        a = np.abs(ref)
        _, ex = np.frexp(np.maximum(a, 1e-38))
        tol = np.ldexp(1.0, ex - 8) + np.ldexp(np.max(a), -16)
        bad = np.abs(got - ref) > tol
        assert not bad.any(), (f"{bad.sum()} bf16 elements off: worst "
                               f"{np.max(np.abs(got - ref)[bad])} vs tol {tol[bad][0]}")
    exact = float(np.mean(bits == bf16_from_f64_vec(ref)))
    print(f"  bf16 outputs bit-equal to the rounded reference: {exact:.5f} of {bits.size}")
    assert exact >= min_exact, f"only {exact:.5f} of bf16 outputs exact"
    return exact


def assert_lora_close(got_bits, oracle_bits, x_bf16, l1_bf16, min_exact=0.999):
    """lora_act from the GPU (fp32 accumulation, one bf16 rounding) vs the oracle (fp64 sum,
    one bf16 rounding): every element lies in [bf16(s - e), bf16(s + e)] with s the exact sum
    and e = K 2^-24 sum_k |x_k l1_jk| the bound of any fp32 summation order (so it equals the
    oracle's value wherever that interval holds no bf16 rounding boundary; where the sum
    cancels to near zero the interval spans several bf16 values), and at least `min_exact`
    of them equal the oracle's."""
    from oracle import bf16_to_f64
    from oracle.construct import bf16_from_f64_vec
    x = bf16_to_f64(x_bf16)
    l1 = bf16_to_f64(l1_bf16)
    K = x.shape[1]
    exact = x @ l1.T
    e = K * U32 * (np.abs(x) @ np.abs(l1).T)
    got = bf16_to_f64(got_bits)
    lo = bf16_to_f64(bf16_from_f64_vec(exact - e))
    hi = bf16_to_f64(bf16_from_f64_vec(exact + e))
    bad = (got < lo) | (got > hi)
    assert not bad.any(), f"{bad.sum()} lora_act elements beyond the fp32 error bound"
    frac = float(np.mean(np.asarray(got_bits) == np.asarray(oracle_bits)))
    print(f"  lora_act equal to the oracle: {frac:.5f} of {np.size(got_bits)}")
    assert frac >= min_exact, f"only {frac:.5f} of lora_act equal to the oracle"


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
    nb = bd.svdq_quantize_next_workspace_bytes(cfg, ncfg, M)
    work = torch.empty(nb // 4, dtype=torch.float32, device="cuda:0") if r2 else None
    bd.svdq_gemm_w4a4_packed_quantize_next(cfg, M, apacked, wpacked, lo, l2d, bd_, act, ncfg, si,
                                           l1d, buf, scales, nlora, work)
    return buf, scales, nlora

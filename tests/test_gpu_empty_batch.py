"""Every compute entry point with M = 0 token rows: the call succeeds, launches nothing and
leaves every buffer it was given untouched (each holds a sentinel byte pattern before and
after).  Covers the nibble calls (INT4 and NVFP4), the packed calls with and without a K-split
workspace, the allocation-free call, the next-layer quantizer and the AWQ GEMV."""
import pytest
import torch

pytestmark = pytest.mark.gpu

gu = pytest.importorskip("gpu_util")
import bit_diffusion_amd as bd  # noqa: E402

SENT = 0x5A


def buf(nbytes):
    """A 256-byte-aligned device buffer of at least nbytes, filled with the sentinel."""
    return torch.full((max(int(nbytes), 256),), SENT, dtype=torch.uint8, device="cuda:0")


def test_empty_batch_every_entry_point():
    K, N, r = 256, 192, 16
    cfg = bd.LayerCfg.make(K, N, r)
    ncfg = bd.LayerCfg.make(N, 128, r)
    fcfg = bd.LayerCfg.make(K, N, r, "nvfp4")
    bufs = []

    def b(nbytes):
        t = buf(nbytes)
        bufs.append(t)
        return t

    x, si, l1 = b(2 * K), b(4 * K), b(2 * r * K)
    codes, scales, lora = b(K // 2), b(4 * K // 64), b(2 * r)
    wcodes, wscales, l2, bias = b(N * K // 2), b(4 * N * K // 64), b(2 * N * r), b(2 * N)
    out = b(4 * N)
    fsc, fwsc = b(K // 16), b(N * K // 16)
    bd.svdq_quantize_act(cfg, 0, x, si, l1, 1.0, codes, scales, lora)
    bd.svdq_quantize_act(fcfg, 0, x, si, l1, 0.5, codes, fsc, lora)
    for act in (bd.SVDQ_ACT_NONE, bd.SVDQ_ACT_GELU_TANH):
        for dt in (bd.SVDQ_DT_F32, bd.SVDQ_DT_BF16):
            bd.svdq_gemm_w4a4(cfg, 0, codes, scales, 1.0, wcodes, wscales, 1.0, lora, l2, bias, act, dt, out)
            bd.svdq_gemm_w4a4(fcfg, 0, codes, fsc, 0.5, wcodes, fwsc, 0.25, lora, l2, bias, act, dt, out)

    l1p = b(bd.svdq_prepacked_l1_bytes(cfg))
    apk = b(bd.svdq_act_packed_bytes(cfg, 256))
    wpk = b(bd.svdq_prepacked_weight_bytes(cfg))
    assert bd.svdq_act_packed_bytes(cfg, 0) == 0
    bd.svdq_quantize_act_packed(cfg, 0, x, si, l1p, apk, scales, lora)
    bd.svdq_pack_act(cfg, 0, codes, scales, apk)
    ws = b(1024)
    assert bd.svdq_gemm_w4a4_packed_workspace_bytes(cfg, 0, bd.SVDQ_ACT_NONE, bd.SVDQ_DT_F32) == 0
    for dt in (bd.SVDQ_DT_F32, bd.SVDQ_DT_BF16):
        bd.svdq_gemm_w4a4_packed(cfg, 0, apk, wpk, lora, l2, bias, bd.SVDQ_ACT_NONE, dt, out)
        bd.svdq_gemm_w4a4_packed_ws(cfg, 0, apk, wpk, lora, l2, bias, bd.SVDQ_ACT_NONE, dt, out, ws, 1024)
        bd.svdq_gemm_w4a4_packed_noalloc(cfg, 0, apk, wpk, lora, l2, bias, bd.SVDQ_ACT_NONE, dt, out)
    nl1, napk, nsc, nlora = b(2 * r * N), b(bd.svdq_act_packed_bytes(ncfg, 256)), b(4 * N // 64), b(2 * r)
    work = b(max(bd.svdq_quantize_next_workspace_bytes(cfg, ncfg, 0), 256))
    bd.svdq_gemm_w4a4_packed_quantize_next(cfg, 0, apk, wpk, lora, l2, bias, bd.SVDQ_ACT_GELU_TANH,
                                           ncfg, si, nl1, napk, nsc, nlora, work)
    aq, asz = b(N * K // 2), b(2 * N * K // 64)
    bd.awq_gemm_w4a16(0, K, N, 64, x, aq, asz, asz, bias, bd.SVDQ_DT_F32, out)
    bd.svdq_calib_absmax(0, K, x, b(4 * K))

    torch.cuda.synchronize()
    for t in bufs:
        assert bool((t == SENT).all()), "an M = 0 call wrote to one of its buffers"

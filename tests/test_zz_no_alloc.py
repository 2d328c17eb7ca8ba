"""svdq_gemm_w4a4_packed_noalloc, the packed GEMM whose K-split partial tiles live in the
library's own device array (for callers that cannot allocate), against
svdq_gemm_w4a4_packed_ws with a caller workspace of the queried size: the same bits, on two
calls in a row, the second on a smaller input, and a third that does not split; the split
output also against the oracle within the fp32 error bound."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import oracle
import synth

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _case(rng, M, N, K, r):
    ca = synth.random_packed_nibbles(rng, M, K)
    sa = rng.uniform(0.01, 0.5, (M, K // 64)).astype(np.float32)
    cw = synth.random_packed_nibbles(rng, N, K)
    sw = rng.uniform(0.001, 0.05, (N, K // 64)).astype(np.float32)
    lora = synth.random_bf16(rng, (M, r), 1.0)
    l2 = synth.random_bf16(rng, (N, r), 0.1)
    b = synth.random_bf16(rng, (N,), 0.3)
    return ca, sa, cw, sw, lora, l2, b


def _run(fn_name, cfg, M, ap, wp, lo, l2, b, N):
    out = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    if fn_name == "ws":
        nb = bd.svdq_gemm_w4a4_packed_workspace_bytes(cfg, M, bd.SVDQ_ACT_NONE, bd.SVDQ_DT_F32)
        ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda:0")
        bd.svdq_gemm_w4a4_packed_ws(cfg, M, ap, wp, lo, l2, b, bd.SVDQ_ACT_NONE, bd.SVDQ_DT_F32, out,
                                    ws, nb)
        torch.cuda.synchronize()
        del ws
    else:
        bd.svdq_gemm_w4a4_packed_noalloc(cfg, M, ap, wp, lo, l2, b, bd.SVDQ_ACT_NONE,
                                         bd.SVDQ_DT_F32, out)
        torch.cuda.synchronize()
    return gu.host(out)


def test_noalloc_matches_workspace_call():
    K, r = 1024, 32
    rng = np.random.default_rng(4242)
    for M, N, splits in ((4352, 3072, True), (4300, 2998, True), (300, 500, False)):
        print(f"noalloc gemm M={M} N={N} K={K} r={r} split={splits}", flush=True)
        ca, sa, cw, sw, lora, l2, b = _case(rng, M, N, K, r)
        cfg = bd.LayerCfg.make(K, N, r)
        nb = bd.svdq_gemm_w4a4_packed_workspace_bytes(cfg, M, bd.SVDQ_ACT_NONE, bd.SVDQ_DT_F32)
        assert (nb > 0) == splits
        ap = gu.pack_act(ca, sa, K)
        wp = gu.prepack(cw, sw, K, N)
        lo, l2d, bd_ = gu.dev(lora), gu.dev(l2), gu.dev(b)
        y_na = _run("noalloc", cfg, M, ap, wp, lo, l2d, bd_, N)
        y_ws = _run("ws", cfg, M, ap, wp, lo, l2d, bd_, N)
        assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), "noalloc differs"
        mi = rng.integers(max(0, M - 300), M, 400)
        ni = rng.integers(0, N, 400)
        ref = oracle.gemm_w4a4_int4_at(mi, ni, ca, sa, cw, sw, lora, l2, b)
        assert gu.rel_fro(y_na[mi, ni], ref) <= 1e-3
        cond = gu.int4_cond(ca, sa, cw, sw, lora, l2, b, mi, ni)
        gu.assert_f32_within(y_na[mi, ni], ref, cond, gu.int4_nround(K, r))


def test_noalloc_rejects_bad_arguments():
    cfg = bd.LayerCfg.make(1024, 3072, 32)
    out = torch.empty((16, 3072), dtype=torch.float32, device="cuda:0")
    with pytest.raises(bd.SvdqError):
        bd.svdq_gemm_w4a4_packed_noalloc(cfg, 16, None, None, None, None, None, 0, 0, out)
    with pytest.raises(bd.SvdqError):
        bd.svdq_gemm_w4a4_packed_noalloc(bd.LayerCfg.make(1024, 3072, 32, "nvfp4"), 16, out, out,
                                         out, out, None, 0, 0, out)

"""The packed linear (activation kernel + GEMM) captured in a HIP graph: every replay, with
eager work and synchronizations between replays, gives bit for bit what eager launches
give (every kernel sums in a fixed order, the K split of a nearly empty last round of
tiles included).  The benchmark times such a replay."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import synth

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _linear(M, K, N, r, out_dtype, seed, split=False):
    rng = np.random.default_rng(seed)
    dev = "cuda:0"
    x = gu.dev(synth.random_bf16(rng, (M, K), 1.0))
    si = gu.dev(rng.uniform(0.5, 2.0, K).astype(np.float32))
    cw = synth.random_packed_nibbles(rng, N, K)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    wpk = gu.prepack(cw, sw, K, N)
    l1p = gu.prepack_l1(synth.random_bf16(rng, (r, K), 0.05), K)
    l2 = gu.dev(synth.random_bf16(rng, (N, r), 0.1))
    b = gu.dev(synth.random_bf16(rng, (N,), 0.3))
    cfg = bd.LayerCfg.make(K, N, r)
    apk = torch.empty(bd.svdq_act_packed_bytes(cfg, M), dtype=torch.uint8, device=dev)
    lora = torch.empty((M, r), dtype=torch.int16, device=dev)
    out = torch.empty((M, N), dtype=torch.float32 if out_dtype == bd.SVDQ_DT_F32 else torch.int16, device=dev)
    nb = bd.svdq_gemm_w4a4_packed_workspace_bytes(cfg, M, bd.SVDQ_ACT_NONE, out_dtype) if split else 0
    assert not split or nb > 0, "this shape is expected to split"
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)

    def step(stream):
        sp = stream.cuda_stream
        bd.svdq_quantize_act_packed(cfg, M, x, si, l1p, apk, None, lora, sp)
        bd.svdq_gemm_w4a4_packed_ws(cfg, M, apk, wpk, lora, l2, b, bd.SVDQ_ACT_NONE, out_dtype, out,
                                    ws, nb, sp)
    return step, out


@pytest.mark.parametrize("M,K,N,out_dtype,split", [
    (1000, 1024, 960, 1, False),     # bf16 out
    (700, 512, 500, 0, False),       # fp32 out, one round of tiles
    (4352, 1024, 3072, 0, True),     # fp32 out, last round split over K (workspace)
])
def test_packed_linear_graph_replays(M, K, N, out_dtype, split):
    print(f"graph replay M={M} K={K} N={N} out_dtype={out_dtype} split={split}", flush=True)
    step, out = _linear(M, K, N, 32, out_dtype, 950 + M, split)
    cur = torch.cuda.current_stream()
    step(cur)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.synchronize()
    for k in range(3):
        out.zero_()                        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k} differs from the eager launch"
        step(cur)                          # and an eager step after it
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


def test_fused_mlp_graph_replays():
    """The MLP with fc2's activation kernel in fc1's epilogue (per-tile partial low-rank sums
    in the workspace, added in a fixed order by a second kernel) captured in a graph: every
    replay's packed codes, scales and fc2's lora_act bit-identical to the eager launch's,
    with eager work (which also dirties the workspace) between the replays."""
    M, K1, N1, r = 700, 512, 768, 32
    rng = np.random.default_rng(960)
    dev = "cuda:0"
    x = gu.dev(synth.random_bf16(rng, (M, K1), 1.0))
    si1 = gu.dev(rng.uniform(0.5, 2.0, K1).astype(np.float32))
    wpk = gu.prepack(synth.random_packed_nibbles(rng, N1, K1),
                     rng.uniform(0.001, 0.05, (N1, K1 // 64)).astype(np.float32), K1, N1)
    l1p = gu.prepack_l1(synth.random_bf16(rng, (r, K1), 0.05), K1)
    l2 = gu.dev(synth.random_bf16(rng, (N1, r), 0.1))
    b = gu.dev(synth.random_bf16(rng, (N1,), 0.3))
    si2 = gu.dev(rng.uniform(0.5, 2.0, N1).astype(np.float32))
    nl1 = gu.dev(synth.random_bf16(rng, (r, N1), 0.05))
    cfg, ncfg = bd.LayerCfg.make(K1, N1, r), bd.LayerCfg.make(N1, 1, r)
    apk = torch.empty(bd.svdq_act_packed_bytes(cfg, M), dtype=torch.uint8, device=dev)
    lora = torch.empty((M, r), dtype=torch.int16, device=dev)
    npk = torch.empty(bd.svdq_act_packed_bytes(ncfg, M), dtype=torch.uint8, device=dev)
    nsc = torch.empty((M, N1 // 64), dtype=torch.float32, device=dev)
    nlora = torch.empty((M, r), dtype=torch.int16, device=dev)
    work = torch.empty(bd.svdq_quantize_next_workspace_bytes(cfg, ncfg, M) // 4, dtype=torch.float32,
                       device=dev)

    def step(stream):
        sp = stream.cuda_stream
        bd.svdq_quantize_act_packed(cfg, M, x, si1, l1p, apk, None, lora, sp)
        bd.svdq_gemm_w4a4_packed_quantize_next(cfg, M, apk, wpk, lora, l2, b, bd.SVDQ_ACT_GELU_TANH,
                                               ncfg, si2, nl1, npk, nsc, nlora, work, sp)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    e_pk, e_sc, e_lo = npk.clone(), nsc.clone(), gu.host(nlora)
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.synchronize()
    for k in range(3):
        npk.zero_()                        # eager work between replays
        nlora.zero_()
        work.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(npk, e_pk), f"replay {k}: packed codes differ"
        assert torch.equal(nsc.view(torch.int32), e_sc.view(torch.int32)), f"replay {k}: scales differ"
        assert np.array_equal(gu.host(nlora), e_lo), f"replay {k}: lora_act differs"


@pytest.mark.parametrize("N,out_dtype", [(6056, 1), (6056, 0), (6050, 1)])
def test_nvfp4_linear_graph_replays(N, out_dtype):
    """The NVFP4 linear (activation kernel + GEMM) with more 256 x 192 tiles (9 x 32) than
    compute units, so each workgroup of the GEMM takes several tiles in turn (with a bf16
    output staged through LDS, N = 6056, the next tile's first stage is copied during the
    current tile's last one), captured in a graph: every replay bit-identical to the eager
    launch, with eager work between the replays."""
    M, K, r = 2100, 512, 32
    print(f"nvfp4 graph replay M={M} K={K} N={N} out_dtype={out_dtype}", flush=True)
    rng = np.random.default_rng(970 + N + out_dtype)
    dev = "cuda:0"
    x = gu.dev(synth.random_bf16(rng, (M, K), 1.0))
    si = gu.dev(rng.uniform(0.5, 2.0, K).astype(np.float32))
    l1 = gu.dev(synth.random_bf16(rng, (r, K), 0.05))
    wc = gu.dev(synth.random_packed_nibbles(rng, N, K))
    ws = gu.dev(rng.integers(0x30, 0x40, (N, K // 16)).astype(np.uint8))
    l2 = gu.dev(synth.random_bf16(rng, (N, r), 0.1))
    b = gu.dev(synth.random_bf16(rng, (N,), 0.3))
    cfg = bd.LayerCfg.make(K, N, r, "nvfp4")
    ac = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    asc = torch.empty((M, K // 16), dtype=torch.uint8, device=dev)
    lora = torch.empty((M, r), dtype=torch.int16, device=dev)
    out = torch.empty((M, N), dtype=torch.float32 if out_dtype == bd.SVDQ_DT_F32 else torch.int16, device=dev)
    Sa, Sw = 0.01, 0.002

    def step(stream):
        sp = stream.cuda_stream
        bd.svdq_quantize_act(cfg, M, x, si, l1, Sa, ac, asc, lora, sp)
        bd.svdq_gemm_w4a4(cfg, M, ac, asc, Sa, wc, ws, Sw, lora, l2, b, bd.SVDQ_ACT_GELU_TANH, out_dtype,
                          out, sp)

    cur = torch.cuda.current_stream()
    step(cur)
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(side)
    torch.cuda.synchronize()
    for k in range(3):
        out.zero_()                        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k} differs from the eager launch"
        step(cur)                          # and an eager step after it
        torch.cuda.synchronize()
        assert torch.equal(out, eager)

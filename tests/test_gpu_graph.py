"""The packed linear (activation kernel + GEMM) captured in a HIP graph: every replay, with
eager work and synchronizations between replays, gives what eager launches give.  The
benchmark times such a replay.  Bit-exact where the GEMM is deterministic; the K-split
shape (fp32 atomics) within fp32 rounding."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import synth

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _linear(M, K, N, r, out_dtype, seed):
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

    def step(stream):
        sp = stream.cuda_stream
        bd.svdq_quantize_act_packed(cfg, M, x, si, l1p, apk, None, lora, sp)
        bd.svdq_gemm_w4a4_packed(cfg, M, apk, wpk, lora, l2, b, bd.SVDQ_ACT_NONE, out_dtype, out, sp)
    return step, out


@pytest.mark.parametrize("M,K,N,out_dtype,exact", [
    (1000, 1024, 960, 1, True),      # bf16 out
    (700, 512, 500, 0, True),        # fp32 out, one round of tiles
    (4352, 1024, 3072, 0, False),    # fp32 out, last round split over K (atomics)
])
def test_packed_linear_graph_replays(M, K, N, out_dtype, exact):
    print(f"graph replay M={M} K={K} N={N} out_dtype={out_dtype}", flush=True)
    step, out = _linear(M, K, N, 32, out_dtype, 950 + M)
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
        if exact:
            assert torch.equal(out, eager), f"replay {k} differs from the eager launch"
        else:
            assert gu.rel_fro(gu.host(out), gu.host(eager)) <= 1e-6, f"replay {k}"
        step(cur)                          # and an eager step after it
        torch.cuda.synchronize()
        if exact:
            assert torch.equal(out, eager)


def test_fused_mlp_graph_replays():
    """The MLP with fc2's activation kernel in fc1's epilogue (the workspace zeroing is a
    fill kernel, the partial low-rank sums fp32 atomics) captured in a graph: every replay's
    packed codes and scales bit-identical to the eager launch's, fc2's lora_act within one
    bf16 ulp, with eager work between the replays."""
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
    work = torch.empty((M, r), dtype=torch.float32, device=dev)

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
        assert gu.bf16_ulp_diff(gu.host(nlora), e_lo).max() <= 1, f"replay {k}: lora_act differs"

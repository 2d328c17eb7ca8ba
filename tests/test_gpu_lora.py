"""GPU parity of svdq_merge_lora (a LoRA adapter through the low-rank branch): the merged
factors bit-exact against the oracle's merge, and the packed linear run at the merged rank
against the oracle (relative Frobenius <= 1e-3), including a rank padded to a multiple of
16, a base rank of 0 and the maximum merged rank 128."""
import numpy as np
import pytest
import torch

import bit_diffusion_amd as bd
import oracle
import synth

pytestmark = pytest.mark.gpu
gu = pytest.importorskip("gpu_util")


def _merge_gpu(K, N, l1, l2, down, up, alpha):
    r = 0 if l1 is None else l1.shape[0]
    rl = down.shape[0]
    ro = bd.svdq_merged_rank(r, rl)
    cfg = bd.LayerCfg.make(K, N, r)
    l1o = torch.empty((ro, K), dtype=torch.int16, device="cuda:0")
    l2o = torch.empty((N, ro), dtype=torch.int16, device="cuda:0")
    bd.svdq_merge_lora(cfg, rl, None if l1 is None else gu.dev(l1), None if l2 is None else gu.dev(l2),
                       gu.dev(down), gu.dev(up), alpha, l1o, l2o)
    torch.cuda.synchronize()
    return gu.host(l1o).view(np.uint16), gu.host(l2o).view(np.uint16)


@pytest.mark.parametrize("K,N,r,rl,alpha", [(192, 200, 16, 8, 0.5), (512, 384, 32, 16, 1.5),
                                            (256, 130, 0, 4, -2.0), (128, 96, 112, 16, 0.25)])
def test_merge_lora_matches_oracle(K, N, r, rl, alpha):
    rng = np.random.default_rng(1300 + K + N + r + rl)
    print(f"merge lora K={K} N={N} r={r} rl={rl}", flush=True)
    l1 = synth.random_bf16(rng, (r, K), 0.05) if r else None
    l2 = synth.random_bf16(rng, (N, r), 0.1) if r else None
    down = synth.random_bf16(rng, (rl, K), 0.05)
    up = synth.random_bf16(rng, (N, rl), 0.1)
    g1, g2 = _merge_gpu(K, N, l1, l2, down, up, alpha)
    o1, o2 = oracle.merge_lora(l1, l2, down, up, alpha)
    assert np.array_equal(g1, o1) and np.array_equal(g2, o2)


@pytest.mark.parametrize("M,K,N,r,rl", [(300, 512, 400, 32, 16), (257, 384, 200, 16, 5)])
def test_packed_linear_with_merged_lora(M, K, N, r, rl):
    rng = np.random.default_rng(1310 + M + rl)
    print(f"packed linear with lora M={M} K={K} N={N} r={r} rl={rl}", flush=True)
    x = synth.random_bf16(rng, (M, K), 1.0)
    si = rng.uniform(0.5, 2.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05)
    l2 = synth.random_bf16(rng, (N, r), 0.1)
    down = synth.random_bf16(rng, (rl, K), 0.05)
    up = synth.random_bf16(rng, (N, rl), 0.1)
    cw = synth.random_packed_nibbles(rng, N, K)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    b = synth.random_bf16(rng, (N,), 0.3)
    g1, g2 = _merge_gpu(K, N, l1, l2, down, up, 0.8)
    buf, _, lora = gu.quantize_packed(x, si, g1)
    y = gu.host(gu.gemm_packed(buf, gu.prepack(cw, sw, K, N), M, K, N, lora, g2, b))
    o1, o2 = oracle.merge_lora(l1, l2, down, up, 0.8)
    oc, os_, ol = oracle.quant_act_int4(x, si, o1)
    ref = oracle.gemm_w4a4_int4(oc, os_, cw, sw, ol, o2, b)
    assert gu.rel_fro(y, ref) <= 1e-3

"""Pins of the oracle's LoRA merge (a LoRA adapter through the SVDQuant low-rank branch):
the merged branch adds, on top of the base layer, the adapter's alpha (x A^T) B^T computed
independently in fp64 from first principles (up to the branch's two bf16 roundings), and
the rank padding contributes exact zeros."""
import numpy as np
import pytest

import oracle
import synth


def _case(rng, M, K, N, r, rl):
    x = synth.random_bf16(rng, (M, K), 1.0)
    si = rng.uniform(0.5, 2.0, K).astype(np.float32)
    l1 = synth.random_bf16(rng, (r, K), 0.05) if r else None
    l2 = synth.random_bf16(rng, (N, r), 0.1) if r else None
    down = synth.random_bf16(rng, (rl, K), 0.05)
    up = synth.random_bf16(rng, (N, rl), 0.1)
    cw = synth.random_packed_nibbles(rng, N, K)
    sw = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    return x, si, l1, l2, down, up, cw, sw


@pytest.mark.parametrize("r,rl,alpha", [(16, 8, 0.5), (32, 16, 2.0), (0, 4, 1.25), (16, 16, -0.75)])
def test_merged_branch_adds_the_adapter_term(r, rl, alpha):
    rng = np.random.default_rng(1200 + r + rl)
    M, K, N = 24, 192, 40
    x, si, l1, l2, down, up, cw, sw = _case(rng, M, K, N, r, rl)
    l1o, l2o = oracle.merge_lora(l1, l2, down, up, alpha)
    ro = (r + rl + 15) // 16 * 16
    assert l1o.shape == (ro, K) and l2o.shape == (N, ro)
    # base layer, and the layer with the merged branch (same codes and scales)
    oc, os_, ol = oracle.quant_act_int4(x, si, l1)
    oc2, os2, ol2 = oracle.quant_act_int4(x, si, l1o)
    assert np.array_equal(oc, oc2) and np.array_equal(os_, os2)
    base = oracle.gemm_w4a4_int4(oc, os_, cw, sw, ol, l2)
    merged = oracle.gemm_w4a4_int4(oc, os_, cw, sw, ol2, l2o)
    # the adapter from first principles: alpha (x A^T) B^T in fp64
    xf = oracle.bf16_to_f64(x)
    term = alpha * (xf @ oracle.bf16_to_f64(down).T) @ oracle.bf16_to_f64(up).T
    diff = merged - base
    # two bf16 roundings (lora_act and alpha B) bound the relative error by ~2 x 2^-9
    assert np.linalg.norm(diff - term) <= 2.0 ** -7 * np.linalg.norm(term)
    # a wrong sign or a dropped alpha would be far off
    assert np.linalg.norm(diff - term) < 0.1 * np.linalg.norm(diff + term)


def test_merge_padding_is_exact_zero_and_base_is_kept():
    rng = np.random.default_rng(1210)
    M, K, N, r, rl = 16, 128, 24, 16, 5
    x, si, l1, l2, down, up, cw, sw = _case(rng, M, K, N, r, rl)
    l1o, l2o = oracle.merge_lora(l1, l2, down, up, 3.0)
    assert l1o.shape[0] == 32
    assert np.array_equal(l1o[:r], l1) and np.array_equal(l2o[:, :r], l2)
    assert np.array_equal(l1o[r:r + rl], down)
    assert not l1o[r + rl:].any() and not l2o[:, r + rl:].any()
    # padded ranks give exact zeros in lora_act; the base ranks are unchanged
    _, _, ol = oracle.quant_act_int4(x, si, l1)
    _, _, ol2 = oracle.quant_act_int4(x, si, l1o)
    assert np.array_equal(ol2[:, :r], ol) and not ol2[:, r + rl:].any()
    # alpha B: exactly the bf16 rounding of the fp32 product (3 x bf16 needs at most 10 bits:
    # checked against the exact product rounded once)
    exact = 3.0 * oracle.bf16_to_f64(up)
    assert np.array_equal(l2o[:, r:r + rl], oracle.bf16_from_f64(exact))

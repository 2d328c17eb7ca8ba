"""Benchmark of the SVDQuant W4A4 linear on one MI355X.

One step = the whole hot path of one linear layer on one batch: the activation kernel
(smoothing, INT4 group quantization, fused low-rank down-projection) followed by the W4A4
GEMM (per-group dequantization, low-rank up-projection, bias), for the DiT attention
projection at 1024x1024 image scale: M = 4096 tokens, K = N = 3072, rank 32, INT4 groups
of 64, bf16 bias, bf16 output.

    python bench.py [--gpus 1] [--steps 50] [--warmup 500] [--no-cpu-baseline] [--only-main]
    python bench.py --copy-calibration      # plain 256 MiB device copies (counter calibration)

The timed region is one replay of a HIP graph that holds exactly `--steps` steps, right
after `--warmup` steps of untimed replays (checked against an eager step); `--reps` more
timed replays give the median, p10 and p90 per step, and the same steps launched eagerly
are reported as `ms_per_step_eager`.

Prints one JSON line.  `value` is TOPS of the linear, counting 2MNK + 2MNr + 2MKr
operations per step (the low-rank branch's flops included, the dense bf16 work the method
avoids not counted), with every input already in HBM.  Inputs rotate through enough copies
(> 256 MB) that each step reads activations and weights from HBM, not from the MI355X's
256 MB last-level cache.  Unless --only-main, the line also carries the secondary paths:
the AWQ W4A16 GEMV of the adaLN modulation (M=2, K=3072, N=18432; GB/s against HBM) and the
NVFP4 fused-QKV linear (M=4096, K=3072, N=9216, rank 32; TOPS against the bf16 and FP4
peaks), and the MLP block (M=4608, 3072 -> 12288 -> 3072, fc1 with GELU and bf16 output
feeding fc2's activation kernel; TOPS), and the attention projection with a rank-16 LoRA
adapter merged into its low-rank branch (eager step time next to ms_per_step_eager).  `roofline.traffic` comes from the HBM byte counters recorded for the GEMM kernel
(profiles/), and is null when the kernel's sources changed since they were taken.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

INT8_PEAK_TOPS = 5000.0   # MI355X dense int8 MFMA, published
BF16_PEAK_TFLOPS = 2500.0
FP4_PEAK_TFLOPS = 10100.0
HBM_PEAK_GBS = 8000.0     # MI355X HBM3E, published
GEMM_SOURCES = ["bit_diffusion_amd/csrc/gemm_int4_fp6.hip", "bit_diffusion_amd/csrc/packed_layout.hpp"]
TRAFFIC_FILE = "profiles/traffic_gemm_w4a4_packed_attn_4096x3072x3072.txt"

M, K, N, R = 4096, 3072, 3072, 32
WORKLOAD = "attn_4096x3072x3072_r32"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=500,
                    help="untimed steps first (the clocks settle over the first tens of ms of load)")
    ap.add_argument("--copies", type=int, default=10,
                    help="rotating input sets (each ~30 MB) to defeat the last-level cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="token rows of the workload the CPU oracle baseline runs")
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="host threads of the CPU baseline (default: the cores this process "
                         "may use, at most 16)")
    ap.add_argument("--single-rows", type=int, default=256,
                    help="token rows the CPU baseline also runs on one thread")
    ap.add_argument("--reps", type=int, default=100,
                    help="timed repetitions behind each median / p10 / p90")
    ap.add_argument("--leg", choices=["awq", "nvfp4", "mlp", "weights", "peaks"], default=None,
                    help="run one secondary leg alone and print its JSON")
    ap.add_argument("--profile", choices=["quant", "gemm", "step", "mlp_fc1", "mlp_fc2", "mlp_q2",
                                          "mlp_fused", "nvfp4", "awq", "peak_fp6", "peak_i8",
                                          "copy"], default=None,
                    help="eager launches of one kernel only (--steps of them after --warmup), "
                         "no timing: the workload a profiler's counters are taken on")
    ap.add_argument("--only-main", action="store_true",
                    help="time only the W4A4 linear (no AWQ / NVFP4 legs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run plain 256 MiB device copies only (for the byte-counter scale)")
    return ap.parse_args()


def sources_hash(paths):
    h = hashlib.sha256()
    for pth in paths:
        with open(os.path.join(ROOT, pth), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per GEMM launch from the recorded counter runs, if they were taken on the
    current GEMM sources (key: value lines; see the file for the commands)."""
    path = os.path.join(ROOT, TRAFFIC_FILE)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("sources_sha256_16") != sources_hash(GEMM_SOURCES):
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration():
    """Plain device-to-device copies of 256 MiB: FETCH_SIZE / WRITE_SIZE of these dispatches
    against the known 268,435,456 bytes each way give the counters' byte scale."""
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_each_way": n, "copies": 10}), flush=True)


def time_launches(fn, n, stream):
    """Mean per-call time (ms) of n calls fn(i) on `stream`, events on that stream."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def launch_stats(fn, batch, reps):
    """Per-call times (ms) of fn(i, stream_handle): `batch` calls captured once into a HIP
    graph on a side stream, the graph replayed `reps` times with an event pair around each
    replay on that stream (so each sample is the mean of `batch` back-to-back calls and the
    events' own latency is spread over them).  Returns mean, median, p10, p90 (ms per call)
    and the counts."""
    import torch
    cs = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(g, stream=cs):
            for i in range(batch):
                fn(i, cs.cuda_stream)
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        g.replay()                      # the first replay uploads the graph
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    with torch.cuda.stream(cs):
        for a, b in ev:
            a.record(cs)
            g.replay()
            b.record(cs)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) / batch for a, b in ev])
    return {"mean": round(float(t.mean()), 5), "median": round(float(np.median(t)), 5),
            "p10": round(float(np.percentile(t, 10)), 5),
            "p90": round(float(np.percentile(t, 90)), 5), "reps": reps, "batch": batch}


def awq_leg(reps, sp, stream, profile_calls=0):
    """AWQ W4A16 GEMV of the modulation layers: M=2, K=3072, N=18432, 14 rotating weight
    copies (> 400 MB, so every call streams its weights from HBM)."""
    import torch
    import synth
    import bit_diffusion_amd as bd
    Ma, Ka, Na, copies = 2, 3072, 18432, 14
    rng = np.random.default_rng(11)
    dev = "cuda:0"

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    qs = [torch.from_numpy(synth.random_packed_nibbles(rng, Na, Ka)).to(dev) for _ in range(copies)]
    sc = [t16(synth.random_bf16(rng, (Na, Ka // 64), 0.01)) for _ in range(copies)]
    zs = [t16(synth.f32_to_bf16_bits(rng.integers(0, 16, (Na, Ka // 64)).astype(np.float32)))
          for _ in range(copies)]
    x = t16(synth.random_bf16(rng, (Ma, Ka), 1.0))
    b = t16(synth.random_bf16(rng, (Na,), 0.1))
    out = torch.empty((Ma, Na), dtype=torch.float32, device=dev)

    def go(i, st=sp):
        k = i % copies
        bd.awq_gemm_w4a16(Ma, Ka, Na, 64, x, qs[k], sc[k], zs[k], b, bd.SVDQ_DT_F32, out, st)

    for i in range(copies):
        go(i)
    torch.cuda.synchronize()
    if profile_calls:
        for i in range(profile_calls):
            go(i)
        return None
    st = launch_stats(go, 2 * copies, reps)
    ms = st["mean"]
    nbytes = Na * Ka // 2 + 2 * Na * (Ka // 64) * 2 + Ma * Ka * 2 + Na * 2 + Ma * Na * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"workload": "awq_modulation_2x3072x18432", "us_per_call": round(ms * 1e3, 3),
            "us_median": round(st["median"] * 1e3, 3), "us_p10": round(st["p10"] * 1e3, 3),
            "us_p90": round(st["p90"] * 1e3, 3), "reps": reps,
            "bytes": nbytes, "GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def nvfp4_leg(reps, sp, stream, profile_calls=0):
    """NVFP4 fused-QKV linear: activation kernel + GEMM, M=4096, K=3072, N=9216, rank 32."""
    import torch
    import synth
    import bit_diffusion_amd as bd
    Mn, Kn, Nn, Rn = 4096, 3072, 9216, 32
    rng = np.random.default_rng(12)
    dev = "cuda:0"

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    cfg = bd.LayerCfg.make(Kn, Nn, Rn, "nvfp4")
    x = t16(synth.random_bf16(rng, (Mn, Kn), 1.0))
    si = torch.ones(Kn, dtype=torch.float32, device=dev)
    l1 = t16(synth.random_bf16(rng, (Rn, Kn), 0.02))
    l2 = t16(synth.random_bf16(rng, (Nn, Rn), 0.02))
    wc = torch.from_numpy(synth.random_packed_nibbles(rng, Nn, Kn)).to(dev)
    ws = torch.from_numpy(rng.integers(0x30, 0x40, (Nn, Kn // 16)).astype(np.uint8)).to(dev)
    bias = t16(synth.random_bf16(rng, (Nn,), 0.02))
    ac = torch.empty((Mn, Kn // 2), dtype=torch.uint8, device=dev)
    asb = torch.empty((Mn, Kn // 16), dtype=torch.uint8, device=dev)
    lora = torch.empty((Mn, Rn), dtype=torch.int16, device=dev)
    out = torch.empty((Mn, Nn), dtype=torch.int16, device=dev)
    Sa, Sw = 0.002, 0.0005

    def quant(i, st=sp):
        bd.svdq_quantize_act(cfg, Mn, x, si, l1, Sa, ac, asb, lora, st)

    def gemm(i, st=sp):
        bd.svdq_gemm_w4a4(cfg, Mn, ac, asb, Sa, wc, ws, Sw, lora, l2, bias, bd.SVDQ_ACT_NONE,
                          bd.SVDQ_DT_BF16, out, st)

    def go(i, st=sp):
        quant(i, st)
        gemm(i, st)

    go(0)
    torch.cuda.synchronize()
    if profile_calls:
        for i in range(profile_calls):
            go(i)
        return None
    stl = launch_stats(go, 5, reps)
    stg = launch_stats(gemm, 5, reps)
    ms, msg = stl["mean"], stg["mean"]
    ops = 2.0 * Mn * Nn * Kn + 2.0 * Mn * Nn * Rn + 2.0 * Mn * Kn * Rn
    ops_g = 2.0 * Mn * Nn * Kn + 2.0 * Mn * Nn * Rn
    tops = ops / (ms * 1e-3) / 1e12
    tops_g = ops_g / (msg * 1e-3) / 1e12
    return {"workload": "nvfp4_qkv_4096x3072x9216_r32", "ms_per_linear": round(ms, 4),
            "ms_median": stl["median"], "ms_p10": stl["p10"], "ms_p90": stl["p90"], "reps": reps,
            "TOPS": round(tops, 2), "bf16_peak_frac": round(tops / BF16_PEAK_TFLOPS, 4),
            "fp4_peak_frac": round(tops / FP4_PEAK_TFLOPS, 4),
            "gemm_ms": round(msg, 4), "gemm_ms_median": stg["median"], "gemm_TOPS": round(tops_g, 2),
            "gemm_f16_peak_frac": round(tops_g / BF16_PEAK_TFLOPS, 4)}


def mlp_profile(what, calls, sp):
    mlp_leg(0, sp, None, profile=(what, calls))


def mlp_leg(reps, sp, stream, profile=None):
    """DiT MLP block on the packed path (M=4608 tokens, 3072 -> 12288 -> 3072, rank 32):
    fc1 with GELU(tanh) in its epilogue writing bf16, then fc2's activation kernel reads that
    output and fc2 writes fp32 (its nearly empty last round of tiles split over K in the
    workspace); and the same block with fc2's activation kernel fused into fc1's epilogue
    (the bf16 intermediate never stored).  Weights are this library's own quantization of
    bf16 N(0, 0.02) draws; activations bf16 N(0, 1) with 31 outlier channels x50."""
    import torch
    import bit_diffusion_amd as bd
    Mm, K1, N1, Rm = 4608, 3072, 12288, 32
    K2, N2 = N1, K1
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(31)

    def bf16(shape, std):
        return (torch.randn(shape, device=dev, generator=g) * std).to(torch.bfloat16).view(torch.int16)

    def layer(K, N):
        cfg = bd.LayerCfg.make(K, N, Rm)
        cw = bd.LayerCfg.make(K, N, 0)
        w = bf16((N, K), 0.02)
        ones = torch.ones(K, dtype=torch.float32, device=dev)
        wc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        ws = torch.empty((N, K // 64), dtype=torch.float32, device=dev)
        bd.svdq_quantize_act(cw, N, w, ones, None, 1.0, wc, ws, None)
        packed = torch.empty(bd.svdq_prepacked_weight_bytes(cw), dtype=torch.uint8, device=dev)
        bd.svdq_prepack_weight(cw, wc, ws, packed)
        l1 = bf16((Rm, K), 0.02)
        l1p = torch.empty(bd.svdq_prepacked_l1_bytes(cfg), dtype=torch.uint8, device=dev)
        bd.svdq_prepack_l1(cfg, l1, l1p)
        return dict(cfg=cfg, packed=packed, l1=l1, l1p=l1p, l2=bf16((N, Rm), 0.02), bias=bf16((N,), 0.02),
                    si=torch.rand(K, device=dev, generator=g) + 0.5,
                    apk=torch.empty(bd.svdq_act_packed_bytes(cfg, Mm), dtype=torch.uint8, device=dev),
                    lora=torch.empty((Mm, Rm), dtype=torch.int16, device=dev))

    fc1, fc2 = layer(K1, N1), layer(K2, N2)
    x = bf16((Mm, K1), 1.0)
    x.view(torch.bfloat16)[:, torch.randperm(K1, device=dev, generator=g)[:31]] *= 50
    h = torch.empty((Mm, N1), dtype=torch.int16, device=dev)
    y = torch.empty((Mm, N2), dtype=torch.float32, device=dev)
    split_bytes = bd.svdq_gemm_w4a4_packed_workspace_bytes(fc2["cfg"], Mm, bd.SVDQ_ACT_NONE,
                                                           bd.SVDQ_DT_F32)
    split_ws = torch.empty(max(split_bytes, 16), dtype=torch.uint8, device=dev)
    work = torch.empty(bd.svdq_quantize_next_workspace_bytes(fc1["cfg"], fc2["cfg"], Mm) // 4,
                       dtype=torch.float32, device=dev)

    def quant(L, a, st):
        bd.svdq_quantize_act_packed(L["cfg"], Mm, a, L["si"], L["l1p"], L["apk"], None, L["lora"], st)

    def gemm1(i, st=sp):
        bd.svdq_gemm_w4a4_packed(fc1["cfg"], Mm, fc1["apk"], fc1["packed"], fc1["lora"], fc1["l2"],
                                 fc1["bias"], bd.SVDQ_ACT_GELU_TANH, bd.SVDQ_DT_BF16, h, st)

    def gemm2(out, st):
        bd.svdq_gemm_w4a4_packed_ws(fc2["cfg"], Mm, fc2["apk"], fc2["packed"], fc2["lora"], fc2["l2"],
                                    fc2["bias"], bd.SVDQ_ACT_NONE, bd.SVDQ_DT_F32, out, split_ws,
                                    split_bytes, st)

    def go(i, st=sp):
        quant(fc1, x, st)
        gemm1(i, st)
        quant(fc2, h, st)
        gemm2(y, st)

    yf = torch.empty_like(y)

    def fc1_fused(i, st=sp):
        bd.svdq_gemm_w4a4_packed_quantize_next(
            fc1["cfg"], Mm, fc1["apk"], fc1["packed"], fc1["lora"], fc1["l2"], fc1["bias"],
            bd.SVDQ_ACT_GELU_TANH, fc2["cfg"], fc2["si"], fc2["l1"], fc2["apk"], None, fc2["lora"],
            work, st)

    def go_fused(i, st=sp):   # fc2's activation kernel runs inside fc1's GEMM epilogue
        quant(fc1, x, st)
        fc1_fused(i, st)
        gemm2(yf, st)

    go(0)
    go_fused(0)
    torch.cuda.synchronize()
    if profile is not None:
        what, calls = profile
        fn = {"mlp_fc1": gemm1, "mlp_fc2": lambda i: gemm2(y, sp), "mlp_fused": fc1_fused,
              "mlp_q2": lambda i: quant(fc2, h, sp)}[what]
        for i in range(calls):
            fn(i)
        return None
    # the two orders of the same block agree up to the fp32 order of fc2's down-projection
    fused_rel = float((yf - y).double().norm() / y.double().norm())
    if not fused_rel <= 1e-3:
        raise RuntimeError(f"fused MLP differs from the unfused block: rel {fused_rel:.3e}")
    st = launch_stats(go, 3, reps)
    stf = launch_stats(go_fused, 3, reps)
    ms, ms_fused = st["mean"], stf["mean"]
    ms_fc1 = launch_stats(gemm1, 3, reps)["mean"]
    ms_fc1f = launch_stats(fc1_fused, 3, reps)["mean"]
    ms_q2 = launch_stats(lambda i, s_: quant(fc2, h, s_), 3, reps)["mean"]
    ms_fc2 = launch_stats(lambda i, s_: gemm2(y, s_), 3, reps)["mean"]
    ops1 = 2.0 * Mm * N1 * K1 + 2.0 * Mm * N1 * Rm
    ops2 = 2.0 * Mm * N2 * K2 + 2.0 * Mm * N2 * Rm
    ops = ops1 + ops2 + 2.0 * Mm * (K1 + K2) * Rm
    tops = ops / (ms * 1e-3) / 1e12
    q2_bytes = Mm * K2 * 2 + bd.svdq_act_packed_bytes(fc2["cfg"], Mm) + Mm * Rm * 2 + Rm * K2 * 2
    return {"workload": "mlp_4608x3072x12288x3072_r32", "ms_per_mlp": round(ms, 4),
            "ms_median": st["median"], "ms_p10": st["p10"], "ms_p90": st["p90"], "reps": reps,
            "TOPS": round(tops, 2), "pct_of_int8_peak": round(100 * tops / INT8_PEAK_TOPS, 2),
            "fc1_gelu_bf16_gemm_ms": round(ms_fc1, 4),
            "fc1_gelu_bf16_gemm_TOPS": round(ops1 / (ms_fc1 * 1e-3) / 1e12, 2),
            "fc2_quantize_ms": round(ms_q2, 4),
            "fc2_quantize_GBs": round(q2_bytes / (ms_q2 * 1e-3) / 1e9, 1),
            "fc2_gemm_ksplit_ms": round(ms_fc2, 4),
            "fc2_gemm_ksplit_TOPS": round(ops2 / (ms_fc2 * 1e-3) / 1e12, 2),
            "fc2_split_workspace_bytes": split_bytes,
            "ms_per_mlp_fused": round(ms_fused, 4), "fused_ms_median": stf["median"],
            "fused_TOPS": round(ops / (ms_fused * 1e-3) / 1e12, 2),
            "fc1_gemm_quantize_next_ms": round(ms_fc1f, 4),
            "fused_vs_unfused_rel": float(f"{fused_rel:.3e}")}


def weights_leg(steps, sp, stream):
    """Offline weight quantization of the attention projection (N = K = 3072, rank 32):
    calibration absmax over 4096 bf16 tokens, smoothing factors from an fp32 weight, the
    INT4 residual given bf16 top-r factors, and the top-r factorization (block 48, four
    power iterations).
    Algorithmic bytes: calibration reads x; smoothing reads w; the residual reads w, l1,
    l2, smooth_inv and writes the codes and scales."""
    import torch
    import bit_diffusion_amd as bd
    Mc, K, N, Rw = 4096, 3072, 3072, 32
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(41)
    x = (torch.randn((Mc, K), device=dev, generator=g)).to(torch.bfloat16).view(torch.int16)
    w = torch.randn((N, K), device=dev, generator=g) * 0.02
    l1 = (torch.randn((Rw, K), device=dev, generator=g) * 0.05).to(torch.bfloat16).view(torch.int16)
    l2 = (torch.randn((N, Rw), device=dev, generator=g) * 0.05).to(torch.bfloat16).view(torch.int16)
    cfg = bd.LayerCfg.make(K, N, Rw)
    am = torch.zeros(K, dtype=torch.float32, device=dev)
    wam = torch.empty(K, dtype=torch.float32, device=dev)
    si = torch.empty(K, dtype=torch.float32, device=dev)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((N, K // 64), dtype=torch.float32, device=dev)
    calib = lambda i: bd.svdq_calib_absmax(Mc, K, x, am, sp)
    smooth = lambda i: bd.svdq_smoothing_factors(cfg, w, am, wam, si, sp)
    resid = lambda i: bd.svdq_quantize_residual(cfg, w, si, l1, l2, codes, scales, None, sp)
    Bw, It = 48, 4
    omega = torch.randn((K, Bw), device=dev, generator=g)
    f1 = torch.empty((Rw, K), dtype=torch.int16, device=dev)
    f2 = torch.empty((N, Rw), dtype=torch.int16, device=dev)
    ws = torch.empty(bd.svdq_lowrank_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    factor = lambda i: bd.svdq_lowrank_factors(cfg, w, si, omega, Bw, It, f1, f2, None, ws, sp)
    for f in (calib, smooth, resid, factor):
        f(0)
    torch.cuda.synchronize()
    n = max(5, steps // 5)
    ms_c, ms_s, ms_r = (time_launches(f, n, stream) for f in (calib, smooth, resid))
    ms_f = time_launches(factor, 3, stream)
    b_c = Mc * K * 2 + K * 4
    b_s = N * K * 4 + 3 * K * 4
    b_r = N * K * 4 + Rw * K * 2 + N * Rw * 2 + K * 4 + N * K // 2 + N * (K // 64) * 4
    fp64 = 2.0 * N * K * Rw
    return {"workload": "weights_3072x3072_r32_calib4096",
            "calib_absmax_ms": round(ms_c, 4), "calib_absmax_GBs": round(b_c / (ms_c * 1e-3) / 1e9, 1),
            "smoothing_factors_ms": round(ms_s, 4), "smoothing_factors_GBs": round(b_s / (ms_s * 1e-3) / 1e9, 1),
            "quantize_residual_ms": round(ms_r, 4), "quantize_residual_GBs": round(b_r / (ms_r * 1e-3) / 1e9, 1),
            "quantize_residual_fp64_TFLOPs": round(fp64 / (ms_r * 1e-3) / 1e12, 2),
            "lowrank_factors_ms": round(ms_f, 3), "lowrank_block": Bw, "lowrank_iters": It}


def lora_leg(reps, sp, stream, si, sets):
    """The attention projection with a rank-16 LoRA adapter merged into its low-rank branch
    (svdq_merge_lora: rank 32 + 16 = 48), eager launches over the same rotating inputs."""
    import torch
    import bit_diffusion_amd as bd
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(41)
    rl = 16
    ro = bd.svdq_merged_rank(R, rl)
    cfg = bd.LayerCfg.make(K, N, R)
    cfgm = bd.LayerCfg.make(K, N, ro)
    down = (torch.randn((rl, K), device=dev, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    up = (torch.randn((N, rl), device=dev, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
    merged = []
    for s in sets:
        l1m = torch.empty((ro, K), dtype=torch.int16, device=dev)
        l2m = torch.empty((N, ro), dtype=torch.int16, device=dev)
        bd.svdq_merge_lora(cfg, rl, s["l1"], s["l2"], down, up, 0.5, l1m, l2m)
        l1p = torch.empty(bd.svdq_prepacked_l1_bytes(cfgm), dtype=torch.uint8, device=dev)
        bd.svdq_prepack_l1(cfgm, l1m, l1p)
        merged.append(dict(l1p=l1p, l2=l2m, lora=torch.empty((M, ro), dtype=torch.int16, device=dev)))

    def go(i, st=sp):
        s, m = sets[i % len(sets)], merged[i % len(sets)]
        bd.svdq_quantize_act_packed(cfgm, M, s["x"], si, m["l1p"], s["apacked"], s["scales"],
                                    m["lora"], st)
        bd.svdq_gemm_w4a4_packed(cfgm, M, s["apacked"], s["packed"], m["lora"], m["l2"],
                                 s["bias"], bd.SVDQ_ACT_NONE, bd.SVDQ_DT_BF16, s["out"], st)

    for i in range(len(sets)):
        go(i)
    torch.cuda.synchronize()
    st = launch_stats(go, len(sets), reps)
    ms = st["mean"]
    ops = 2.0 * M * N * K + 2.0 * M * N * ro + 2.0 * M * K * ro
    return {"workload": f"attn_4096x3072x3072_r{R}+lora{rl}", "merged_rank": ro,
            "ms_per_step": round(ms, 5), "ms_median": st["median"], "reps": reps,
            "TOPS": round(ops / (ms * 1e-3) / 1e12, 2)}


def make_inputs(copies):
    """Synthetic inputs of the attention-projection workload, on the GPU.

    Activations: the workload's draw (bf16 N(0,1), 31 outlier channels x50).  Smoothing
    factors from the activation and weight column maxima.  The 4-bit residual weights are
    produced by this library's own activation kernel from a synthetic bf16 residual (the
    GEMM's speed does not depend on the code values).  Low-rank factors: bf16 N(0, 0.02), the down-projection factor prepacked once like the weights.
    """
    import torch
    import synth
    import bit_diffusion_amd as bd

    wl = synth.WORKLOADS[1]
    d = synth.draw(wl)
    xb = d.x_bf16
    xmax = np.abs(synth.bf16_bits_to_f32(xb)).max(axis=0).astype(np.float64)
    wmax = np.abs(d.w).max(axis=0)
    lam = np.sqrt(np.where((xmax > 0) & (wmax > 0), xmax / np.maximum(wmax, 1e-30), 1.0))
    smooth_inv = (1.0 / lam).astype(np.float32)
    rng = np.random.default_rng(7)
    dev = "cuda:0"

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    si = torch.from_numpy(smooth_inv).to(dev)
    ones = torch.ones(K, dtype=torch.float32, device=dev)
    resid = synth.f32_to_bf16_bits((d.w * lam[None, :]).astype(np.float32))
    sets = []
    cfg_w = bd.LayerCfg.make(K, N, 0)
    for c in range(copies):
        x = t16(xb) if c == 0 else t16(np.roll(xb, c, axis=0))
        rt = t16(resid if c == 0 else np.roll(resid, c, axis=0))
        wc = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        ws = torch.empty((N, K // 64), dtype=torch.float32, device=dev)
        bd.svdq_quantize_act(cfg_w, N, rt, ones, None, 1.0, wc, ws, None)
        del rt
        packed = torch.empty(bd.svdq_prepacked_weight_bytes(cfg_w), dtype=torch.uint8, device=dev)
        bd.svdq_prepack_weight(cfg_w, wc, ws, packed)
        s = dict(
            x=x, wc=wc, ws=ws, packed=packed,
            l1=t16(synth.random_bf16(rng, (R, K), 0.02)),
            l2=t16(synth.random_bf16(rng, (N, R), 0.02)),
            bias=t16(d.bias_bf16),
            apacked=torch.empty(bd.svdq_act_packed_bytes(cfg_w, M), dtype=torch.uint8, device=dev),
            scales=torch.empty((M, K // 64), dtype=torch.float32, device=dev),
            lora=torch.empty((M, R), dtype=torch.int16, device=dev),
            out=torch.empty((M, N), dtype=torch.int16, device=dev),
        )
        cfg_r = bd.LayerCfg.make(K, N, R)
        s["l1p"] = torch.empty(bd.svdq_prepacked_l1_bytes(cfg_r), dtype=torch.uint8, device=dev)
        bd.svdq_prepack_l1(cfg_r, s["l1"], s["l1p"])
        sets.append(s)
    torch.cuda.synchronize()
    return si, sets, d


def host_cpu():
    """(CPU model name, logical CPUs this process may run on)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        ncpu = len(os.sched_getaffinity(0))
    except AttributeError:
        ncpu = os.cpu_count() or 1
    return model, ncpu


def cpu_baseline(rows, threads, single_rows):
    """The CPU oracle (as it stands: plain scalar C, one call per row block) on the first
    `rows` token rows of the same workload: activation stage + GEMM with the low-rank branch
    and bias.  The rows are cut into `threads` blocks run by as many host threads (the
    oracle's C calls release the interpreter lock), so every core works; the first
    `single_rows` rows also run on one thread, for the per-core figure."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    import synth

    wl = synth.WORKLOADS[1]
    d = synth.draw(wl)
    rng = np.random.default_rng(7)
    xb = np.ascontiguousarray(d.x_bf16[:rows])
    si = np.ones(K, np.float32)
    l1 = synth.random_bf16(rng, (R, K), 0.02)
    l2 = synth.random_bf16(rng, (N, R), 0.02)
    wc = synth.random_packed_nibbles(rng, N, K)
    ws = rng.uniform(0.001, 0.1, (N, K // 64)).astype(np.float32)
    oracle.lib()

    def block(lo, hi):
        c, s, lo_act = oracle.quant_act_int4(np.ascontiguousarray(xb[lo:hi]), si, l1)
        oracle.gemm_w4a4_int4(c, s, wc, ws, lo_act, l2, d.bias_bf16)

    def ops_of(n):
        return 2.0 * n * N * K + 2.0 * n * N * R + 2.0 * n * K * R

    t0 = time.perf_counter()
    block(0, single_rows)
    t1 = time.perf_counter() - t0
    edges = np.linspace(0, rows, threads + 1).astype(int)
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: block(edges[i], edges[i + 1]), range(threads)))
    dt = time.perf_counter() - t0
    model, ncpu = host_cpu()
    return dict(value=ops_of(rows) / dt / 1e12, unit="TOPS", cores=threads, kind="oracle",
                sample=f"{rows} of {M} token rows, full K and N, C oracle on {threads} host "
                       f"threads, {dt:.2f} s wall",
                cpu_model=model, nproc=ncpu,
                single_thread={"value": ops_of(single_rows) / t1 / 1e12, "unit": "TOPS",
                               "rows": single_rows, "seconds": round(t1, 2)})


def peaks_leg(sp, stream):
    """Measured denominators: each MFMA kind of the kernels at its sustained rate (a kernel
    with independent back-to-back MFMAs on every SIMD, operands in registers); plain HBM
    read and copy of 512 MiB (median of 20); and, in the launch mode the kernels are timed in
    (graph replays of back-to-back launches over rotating buffers that defeat the last-level
    cache), a plain read of the AWQ GEMV's bytes and a plain copy moving as many bytes as the
    activation kernel."""
    import torch
    import bit_diffusion_amd as bd
    dev = "cuda:0"
    out = torch.zeros(4, dtype=torch.float32, device=dev)
    names = {0: "fp6_32x32x64", 1: "i8_32x32x32", 2: "bf16_32x32x16", 3: "bf16_32x32x8",
             4: "f16_32x32x16", 5: "fp4_32x32x64"}
    res = {}
    for kind, name in names.items():
        iters = 2048
        bd.svdq_peak_mfma(kind, iters, out, sp)          # warm
        torch.cuda.synchronize()
        best = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ops = bd.svdq_peak_mfma(kind, iters, out, sp)
            e1.record(stream)
            torch.cuda.synchronize()
            best.append(ops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        res[name] = round(float(np.median(best)), 1)

    def big(fn, moved):
        fn()
        torch.cuda.synchronize()
        r = []
        for _ in range(20):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            r.append(moved / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        return round(float(np.median(r)), 1)

    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    copy_gbs = big(lambda: bd.svdq_peak_copy(src, dst, n, sp), 2 * n)
    read_gbs = big(lambda: bd.svdq_peak_read(src, n, out, sp), n)
    del src, dst
    # same size and launch mode as the AWQ GEMV (32,047,104 B read) and the activation
    # kernel (25,165,824 B of x read; the copy moves 2 x 18.7 MB, its 37.4 MB)
    na, nq, nb = 32047104, 37431296 // 2 // 16 * 16, 14
    bufs = [torch.ones(max(na, nq), dtype=torch.uint8, device=dev) for _ in range(nb)]
    outs = [torch.empty(nq, dtype=torch.uint8, device=dev) for _ in range(nb)]
    st_r = launch_stats(lambda i, s_: bd.svdq_peak_read(bufs[i % nb], na, out, s_), 2 * nb, 100)
    st_c = launch_stats(lambda i, s_: bd.svdq_peak_copy(bufs[i % nb], outs[i % nb], nq, s_), 2 * nb, 100)
    del bufs, outs
    return {"mfma_TOPS": res, "copy_GBs": copy_gbs, "read_GBs": read_gbs,
            "read_awq_size_us": round(st_r["mean"] * 1e3, 3),
            "read_awq_size_GBs": round(na / (st_r["mean"] * 1e-3) / 1e9, 1),
            "copy_quant_size_us": round(st_c["mean"] * 1e3, 3),
            "copy_quant_size_GBs": round(2 * nq / (st_c["mean"] * 1e-3) / 1e9, 1)}


def profile_run(what, steps, warmup, sp):
    """Eager launches of one kernel (warmup + steps of them) on the benchmark's inputs."""
    import torch
    import bit_diffusion_amd as bd
    dev = "cuda:0"
    if what in ("quant", "gemm", "step"):
        si, sets, _ = make_inputs(4)
        cfg = bd.LayerCfg.make(K, N, R)

        def quant(s):
            bd.svdq_quantize_act_packed(cfg, M, s["x"], si, s["l1p"], s["apacked"], s["scales"],
                                        s["lora"], sp)

        def gemm(s):
            bd.svdq_gemm_w4a4_packed(cfg, M, s["apacked"], s["packed"], s["lora"], s["l2"],
                                     s["bias"], bd.SVDQ_ACT_NONE, bd.SVDQ_DT_BF16, s["out"], sp)
        for s in sets:
            quant(s)
        fn = {"quant": quant, "gemm": gemm, "step": lambda s: (quant(s), gemm(s))}[what]
        for i in range(warmup + steps):
            fn(sets[i % len(sets)])
    elif what.startswith("mlp"):
        mlp_profile(what, warmup + steps, sp)
    elif what == "nvfp4":
        nvfp4_leg(0, sp, None, profile_calls=warmup + steps)
    elif what == "awq":
        awq_leg(0, sp, None, profile_calls=warmup + steps)
    elif what in ("peak_fp6", "peak_i8"):
        out = torch.zeros(4, dtype=torch.float32, device=dev)
        for _ in range(warmup + steps):
            bd.svdq_peak_mfma(0 if what == "peak_fp6" else 1, 2048, out, sp)
    else:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(warmup + steps):
            bd.svdq_peak_copy(src, dst, n, sp)
    torch.cuda.synchronize()
    print(json.dumps({"profile": what, "launches": warmup + steps}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the linear "
              "shards over tokens with no communication, see the design notes.", file=sys.stderr)
        sys.exit(2)
    import torch
    import bit_diffusion_amd as bd

    if args.copy_calibration:
        copy_calibration()
        return
    assert bd.svdq_check_device(0) == bd.SVDQ_OK, bd.svdq_last_error()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    if args.profile is not None:
        profile_run(args.profile, args.steps, args.warmup, sp)
        return
    if args.leg is not None:   # one leg alone
        legs = {"awq": lambda: awq_leg(args.reps, sp, stream),
                "nvfp4": lambda: nvfp4_leg(args.reps, sp, stream),
                "mlp": lambda: mlp_leg(args.reps, sp, stream),
                "weights": lambda: weights_leg(args.steps, sp, stream),
                "peaks": lambda: peaks_leg(sp, stream)}
        print(json.dumps({args.leg: legs[args.leg]()}), flush=True)
        return
    si, sets, _ = make_inputs(args.copies)
    cfg = bd.LayerCfg.make(K, N, R)

    def quant(s, st=sp):
        bd.svdq_quantize_act_packed(cfg, M, s["x"], si, s["l1p"], s["apacked"], s["scales"],
                                    s["lora"], st)

    def gemm(s, st=sp):
        bd.svdq_gemm_w4a4_packed(cfg, M, s["apacked"], s["packed"], s["lora"], s["l2"],
                                 s["bias"], bd.SVDQ_ACT_NONE, bd.SVDQ_DT_BF16, s["out"], st)

    def step(s, st=sp):
        quant(s, st)
        gemm(s, st)

    for i in range(min(args.warmup, len(sets))):   # first touch of every input set
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # whole-step timing: the `steps` steps captured once into a HIP graph (capturing runs
    # nothing) and replayed, as a denoising loop launches its layers.  The warmup is graph
    # replays back to back (at least `warmup` steps; the first replay also uploads the
    # graph), then one timed replay: exactly `steps` steps between a synchronisation and an
    # event pair on the replaying stream
    cs = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            for i in range(args.steps):
                step(sets[i % len(sets)], cs.cuda_stream)
    torch.cuda.synchronize()
    for _ in range(max(1, -(-args.warmup // args.steps))):
        graph.replay()
    torch.cuda.synchronize()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # the replayed graph computes what eager launches compute (same inputs, deterministic
    # kernels): the last graph step on set j against one eager step on it
    j = (args.steps - 1) % len(sets)
    from_graph = sets[j]["out"].clone()
    step(sets[j])
    torch.cuda.synchronize()
    if not torch.equal(from_graph, sets[j]["out"]):
        raise RuntimeError("graph replay and eager launch disagree")

    # eager launches of the same steps, for reference
    ev0.record(stream)
    for i in range(args.steps):
        step(sets[i % len(sets)])
    ev1.record(stream)
    torch.cuda.synchronize()
    ms_eager = ev0.elapsed_time(ev1) / args.steps

    # the spread: `reps` more timed replays of the same graph
    reps_t = []
    for _ in range(args.reps):
        ev0.record(stream)
        graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        reps_t.append(ev0.elapsed_time(ev1) / args.steps)
    reps_t = np.array(reps_t)

    # per-kernel timing: each kernel alone, `steps` launches back to back over the rotating
    # input sets captured in a graph, replayed `reps` times with an event pair around each
    # replay on the launching stream
    st_q = launch_stats(lambda i, st: quant(sets[i % len(sets)], st), args.steps, args.reps)
    st_g = launch_stats(lambda i, st: gemm(sets[i % len(sets)], st), args.steps, args.reps)

    ops_gemm = 2.0 * M * N * K + 2.0 * M * N * R
    ops_total = ops_gemm + 2.0 * M * K * R
    value = ops_total / (ms_step * 1e-3) / 1e12
    gemm_tops = ops_gemm / (st_g["mean"] * 1e-3) / 1e12
    # read x, smooth_inv, L1; write 6-bit codes + a 4-byte scale word per (row, group), the
    # fp32 scales and lora_act
    quant_bytes = (M * K * 2 + K * 4 + R * K * 2 + M * K * 3 // 4 + M * (K // 64) * 8
                   + M * R * 2)
    quant_gbs = quant_bytes / (st_q["mean"] * 1e-3) / 1e9
    traffic = recorded_traffic()
    peaks = peaks_leg(sp, stream)
    mfma_meas = peaks["mfma_TOPS"]

    out = {
        "metric": "W4A4+low-rank r32 linear TOPS @4096x3072x3072; % of int8 MFMA peak",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "ms_per_step_stats": {"median": round(float(np.median(reps_t)), 5),
                              "p10": round(float(np.percentile(reps_t, 10)), 5),
                              "p90": round(float(np.percentile(reps_t, 90)), 5),
                              "reps": args.reps, "steps_per_rep": args.steps},
        "ms_per_step_eager": round(ms_eager, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int4",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "M": M, "K": K, "N": N, "rank": R, "group": 64,
                   "out_dtype": "bf16", "bias": True, "pct_of_int8_peak":
                   round(100 * value / INT8_PEAK_TOPS, 2)},
        "roofline": {"bound": "mfma", "achieved": round(gemm_tops, 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TOP/s", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic, "kernel": "svdq_gemm_w4a4_packed (int4 as FP6 on the MFMA)",
                     "ms_per_launch": st_g["mean"], "launch_stats": st_g,
                     "frac_of_fp6_peak": round(gemm_tops / FP4_PEAK_TFLOPS, 4),
                     "measured_peaks_TOPS": {"i8": mfma_meas["i8_32x32x32"],
                                             "fp6": mfma_meas["fp6_32x32x64"]},
                     "frac_of_measured_i8": round(gemm_tops / mfma_meas["i8_32x32x32"], 4)},
        "kernels": {
            "quantize_act_ms": st_q["mean"],
            "quantize_act_stats": st_q,
            "quantize_act_GBs": round(quant_gbs, 1),
            "quantize_act_hbm_frac": round(quant_gbs / HBM_PEAK_GBS, 4),
            "quantize_act_copy_frac": round(quant_gbs / peaks["copy_GBs"], 4),
            "quantize_act_frac_of_same_size_copy": round(quant_gbs / peaks["copy_quant_size_GBs"], 4),
            "gemm_ms": st_g["mean"],
            "gemm_TOPS": round(gemm_tops, 2),
        },
        "peaks_measured": peaks,
    }
    if not args.only_main:
        out["awq"] = awq_leg(args.reps, sp, stream)
        out["awq"]["read_frac"] = round(out["awq"]["GBs"] / peaks["read_GBs"], 4)
        out["awq"]["frac_of_same_size_read"] = round(out["awq"]["GBs"] / peaks["read_awq_size_GBs"], 4)
        out["nvfp4"] = nvfp4_leg(args.reps, sp, stream)
        out["mlp"] = mlp_leg(args.reps, sp, stream)
        out["lora"] = lora_leg(args.reps, sp, stream, si, sets)
        out["weights"] = weights_leg(args.steps, sp, stream)
    if not args.no_cpu_baseline:
        model, ncpu = host_cpu()
        threads = args.cpu_threads or max(1, min(16, ncpu))
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows, threads, args.single_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the differential-attention hot path on one MI355X.

A step is one pass of the path over the V1 prefill workload (B=4, H=16, N=2048, d=64, dv=128,
causal, RMSNorm * (1 - lambda_init) epilogue): lambda from its re-parameterisation and the fused
forward, one library call and one kernel (diffattn_fwd_lambda). Inputs are synthetic (seeded)
and resident in HBM before timing starts. Prints ONE JSON line on stdout; progress goes to
stderr.

Also measured in the same run (reported under "secondary"): the 32K-token prefill with a planted
needle, the 64K-entry V1 decode and the V2 decode, each also on a paged cache (GB/s against HBM),
the V2 GQA prefill (lambda given and from its logits), the V1 backward on the main workload, the
V2 backward on the V2 prefill workload, the main workload with fp8 score operands; and the fp64
oracle on a bounded sample of the main workload, timed on the host cores ("cpu_baseline").

Throughput counts algorithmic work only: 768 flop per visible (query, key) pair for V1 (two
QK^T products of width 64 and two PV products of width 128), 512 per visible pair and query head
for V2, and for decode the bytes of the cache read once (V1: K1, K2 and V, 512 B per cached token
per head; V2: K and V, 512 B per cached token per KV head, shared by the group's query heads).
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "diff-attn fwd TFLOP/s (bf16, N=2K/32K) + decode GB/s; % of MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
FLOP_PER_PAIR_V1 = 768
# the work of ordinary attention on the same pairs (one QK^T of width 64, one PV of width 128),
# printed beside the method's own for transparency; never the metric
FLOP_PER_PAIR_V1_NAIVE_EQ = 512
FLOP_PER_PAIR_V2 = 512
# backward: recomputed scores (2 x 2d), dP = go V^T (2 dv), dV (2 dv), dK and dQ of both maps
# (2 x 2d each): 1280 per visible pair at d = 64, dv = 128
FLOP_PER_PAIR_V1_BWD = 1280
# V2 backward, per visible pair and query head at d = 128: recomputed scores (2d), dQ (2d), dK
# (2d), and dP and dV (2d each per pair of heads, so d per head)
FLOP_PER_PAIR_V2_BWD = 1024
PAGE_SIZE = 256                # tokens per page of the paged decode legs
DECODE_BYTES_PER_TOKEN = 2 * (64 + 64 + 128)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def causal_pairs(n):
    return n * (n + 1) // 2


def kernel_source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "differential_softmax_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# the sources each forward build compiles (short keys: the default schedule; 4096 keys and more:
# the max-ilp build of the same kernels)
FWD_SOURCES = ["fwd_mfma_kernel.hpp", "fwd_mfma.hip", "mfma_tile.hpp", "common.hpp"]
FWD_LONG_SOURCES = ["fwd_mfma_kernel.hpp", "fwd_mfma_long.hip", "mfma_tile.hpp", "common.hpp"]


def load_traffic(name, files):
    """HBM traffic per launch from committed rocprofv3 PMC summaries, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash(files):
        return None
    return t.get("hbm_bytes_per_launch")


def warm_until_stable(fn, floor, torch, min_s=0.5, max_s=5.0, batch=20, tol=0.02):
    """Launch fn at least `floor` times, then in batches of `batch` until at least `min_s` seconds
    have passed and two consecutive batches agree within `tol` (or `max_s` passed), so that the
    timed launches that follow run on a GPU at its steady clock. Returns the launch count."""
    for _ in range(floor):
        fn()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    prev, n = None, floor
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(batch):
            fn()
        e1.record()
        torch.cuda.synchronize()
        n += batch
        avg = e0.elapsed_time(e1) / batch
        elapsed = time.perf_counter() - t_start
        if elapsed >= max_s or (elapsed >= min_s and prev is not None and abs(avg - prev) <= tol * prev):
            return n
        prev = avg


def time_launches(fn, torch, samples=50, per=1):
    """Device time per call of fn on the current stream: `samples` samples, each the mean of `per`
    back-to-back calls between two HIP events (so the events' own cost is spread over `per`
    calls). Returns the mean, median and min over the samples, in ms."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for a, b in evs:
        a.record()
        for _ in range(per):
            fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) / per for a, b in evs)
    return {"mean": statistics.fmean(ms), "median": statistics.median(ms), "min": ms[0]}


def measure(fn, torch, label, samples=50, target_ms=2.0, floor=3, min_s=0.2):
    """Warm fn up until its time is steady, then time it with `per` chosen so a sample lasts about
    target_ms. Logs the call counts under `label`, so that a kernel trace of the run can be split
    into untimed and timed launches."""
    n_warm = warm_until_stable(fn, floor, torch, min_s=min_s, max_s=3.0, batch=4)
    t = time_launches(fn, torch, samples=3, per=1)
    per = max(1, min(50, int(round(target_ms / max(t["median"], 1e-3)))))
    r = time_launches(fn, torch, samples=samples, per=per)
    r["per"] = per
    r["samples"] = samples
    log(f"[bench]   calls of {label}: {n_warm + 3} untimed, then {samples} x {per} timed")
    return r


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def head_major_f64(t):
    """A [B, N, H, dim] tensor as a float64 host array of the same shape whose (b, :, h) slices are
    contiguous, so the oracle reads each head without a copy (layout only; no arithmetic)."""
    import torch
    return t.permute(0, 2, 1, 3).contiguous().to(torch.float64).cpu().numpy().transpose(0, 2, 1, 3)


def sample_rows(n, rng, extra=48):
    """Row sample of a causal prefill: the last row (it sees every key), the rows at 32-, 64- and
    128-row tile boundaries near the start and the middle, and `extra` seeded random rows."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, n // 2 - 1, n // 2, n - 2, n - 1}
    rows = sorted(r for r in fixed if 0 <= r < n)
    rows += sorted(int(x) for x in rng.choice(n, size=extra, replace=False))
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20,
                    help="minimum warm-up launches; warm-up then continues until the launch time is steady")
    ap.add_argument("--secondary", default="32k,decode,v2,v2decode,bwd,v2bwd,fp8",
                    help="comma list of extra workloads to time (32k, decode, v2, v2decode, bwd, v2bwd, fp8) or 'none'")
    ap.add_argument("--secondary-samples", type=int, default=50,
                    help="timing samples per secondary workload (median and min reported)")
    ap.add_argument("--cpu-baseline", type=int, default=1, help="time the fp64 oracle on a sample (1) or not (0)")
    ap.add_argument("--copy-calibration", type=int, default=1,
                    help="run a 1 GiB device copy (reference kernel for HBM counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} (WORLD_SIZE {world}) is not supported: "
              "the differential-attention path here has no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import differential_softmax_attention_amd as da
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = da.lib()

    # ---------------- main workload: V1 prefill 2K ----------------
    cfg = W.V1_PREFILL_2K
    log(f"[bench] generating inputs: {cfg.name}")
    x = W.v1_inputs(cfg, device=dev)
    vecs = [x[k].to(dev).contiguous() for k in ("lq1", "lk1", "lq2", "lk2")]
    lam = torch.empty(cfg.H, dtype=torch.float32, device=dev)
    out = torch.empty((cfg.B, cfg.N, cfg.H, cfg.dv), dtype=torch.bfloat16, device=dev)
    li = da.lambda_init(cfg.layer)
    stream = torch.cuda.current_stream(dev).cuda_stream
    # marshal the C-ABI arguments once; a step is one library call, diffattn_fwd_lambda: lambda
    # from its re-parameterisation and the fused forward in one kernel
    step_args = (da.DIFFATTN_BF16, *(da._t4(x[k]) for k in ("q1", "q2", "k1", "k2", "v")), cfg.B, cfg.H,
                 cfg.N, cfg.N, cfg.d, cfg.dv, *(v.data_ptr() for v in vecs), cfg.d, cfg.layer, lam.data_ptr(), 1,
                 da.EPI_RMSNORM_SCALE, None, 1e-5, 0.0, da._t4(out), stream)

    def fwd_step():
        da._check(L.diffattn_fwd_lambda(*step_args))

    # warm-up: at least --warmup launches, then until the launch time is steady (two 20-launch
    # batches within 2 %, at least 0.5 s), so the timed steps do not run on a cold GPU
    n_warm = warm_until_stable(fwd_step, args.warmup, torch)
    log(f"[bench] warm-up: {n_warm} launches")

    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd_step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # the fused kernel alone, after the timed steps: 50 samples of 10 back-to-back launches, each
    # sample between two HIP events on the launch stream; median and min over the samples
    kt = time_launches(fwd_step, torch, samples=50, per=10)
    flops = FLOP_PER_PAIR_V1 * cfg.B * cfg.H * causal_pairs(cfg.N)
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kt["median"] * 1e-3) / 1e12
    log(f"[bench] step {ms_per_step * 1e3:.1f} us; fused forward kernel median {kt['median'] * 1e3:.1f} us, "
        f"min {kt['min'] * 1e3:.1f} us, mean {kt['mean'] * 1e3:.1f} us -> {achieved:.1f} TFLOP/s")
    traffic = load_traffic("v1_prefill_2k", FWD_SOURCES)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded torch generators; iid N(0,1) inputs, lambda vectors N(0, 0.1^2))",
        "config": {"workload": cfg.name, "batch": cfg.B, "heads": cfg.H, "seq_len": cfg.N, "d": cfg.d,
                   "dv": cfg.dv, "causal": True, "epilogue": "rmsnorm*(1-lambda_init)", "layer": cfg.layer,
                   "step": "diffattn_fwd_lambda (lambda re-parameterisation and the fused forward, one kernel)",
                   "flop_per_step": flops, "flop_per_visible_pair": FLOP_PER_PAIR_V1,
                   "naive_equivalent_TFLOP/s": round(value * FLOP_PER_PAIR_V1_NAIVE_EQ / FLOP_PER_PAIR_V1, 2),
                   "naive_equivalent_flop_per_visible_pair": FLOP_PER_PAIR_V1_NAIVE_EQ},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "fwd_mfma_kernel<64,V1,causal,epilogue,lambda in-kernel>",
                     "kernel_median_us": round(kt["median"] * 1e3, 2),
                     "kernel_min_us": round(kt["min"] * 1e3, 2),
                     "kernel_avg_us": round(kt["mean"] * 1e3, 2),
                     "kernel_timing": "50 samples, each 10 back-to-back launches between two HIP events on "
                                      "the launch stream, after the timed steps; achieved = flop / median",
                     "warmup_launches": n_warm},
    }
    del x

    # ---------------- secondary workloads ----------------
    secondary = {}
    which = [] if args.secondary == "none" else args.secondary.split(",")
    if "32k" in which:
        c3 = W.V1_PREFILL_32K
        log(f"[bench] {c3.name}")
        x3 = W.v1_inputs(c3, device=dev)
        lam3 = da.diffattn_lambda(*(x3[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), c3.layer)
        o3 = torch.empty((c3.B, c3.N, c3.H, c3.dv), dtype=torch.bfloat16, device=dev)
        f3 = lambda: da.diffattn_fwd(x3["q1"], x3["q2"], x3["k1"], x3["k2"], x3["v"], lam3, causal=True,
                                     epilogue=True, lambda_init_value=da.lambda_init(c3.layer), out=o3)
        f3()
        torch.cuda.synchronize()
        _r = measure(f3, torch, "v1_prefill_32k", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        fl3 = FLOP_PER_PAIR_V1 * c3.B * c3.H * causal_pairs(c3.N)
        tf = fl3 / (avg * 1e-3) / 1e12
        secondary["v1_prefill_32k"] = {"workload": c3.name, "kernel_median_ms": round(avg, 4),
                                       "kernel_min_ms": round(mn, 4), "flop": fl3, "TFLOP/s": round(tf, 2),
                                       "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                       "traffic": load_traffic("v1_prefill_32k", FWD_LONG_SOURCES)}
        log(f"[bench]   {avg:.3f} ms -> {tf:.1f} TFLOP/s")
        del x3, o3
    if "v2" in which:
        c5 = W.V2_GQA_8K
        log(f"[bench] {c5.name}")
        x5 = W.v2_inputs(c5, device=dev)
        o5 = torch.empty((c5.B, c5.N, c5.hq // 2, c5.d), dtype=torch.bfloat16, device=dev)
        f5 = lambda: da.diffattn_v2_fwd(x5["q"], x5["k"], x5["v"], x5["lam"], causal=True, out=o5)
        f5()
        torch.cuda.synchronize()
        _r = measure(f5, torch, "v2_gqa_8k", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        fl5 = FLOP_PER_PAIR_V2 * c5.B * c5.hq * causal_pairs(c5.N)
        tf = fl5 / (avg * 1e-3) / 1e12
        secondary["v2_gqa_8k"] = {"workload": c5.name, "kernel_median_ms": round(avg, 4), "kernel_min_ms": round(mn, 4),
                                  "flop": fl5, "TFLOP/s": round(tf, 2),
                                  "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "traffic": load_traffic("v2_gqa_8k", FWD_LONG_SOURCES)}
        log(f"[bench]   {avg:.3f} ms -> {tf:.1f} TFLOP/s")
        # lambda from its logits inside the kernel (sigmoid per query row)
        z5 = W.lambda_logits((c5.B, c5.N, c5.hq // 2), seed=c5.seed + 2000, device=dev)
        fz = lambda: da.diffattn_v2_fwd(x5["q"], x5["k"], x5["v"], z5, causal=True, out=o5, lam_logits=True)
        fz()
        torch.cuda.synchronize()
        _r = measure(fz, torch, "v2_gqa_8k_logits", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        tf = fl5 / (avg * 1e-3) / 1e12
        secondary["v2_gqa_8k"]["lam_logits_kernel_median_ms"] = round(avg, 4)
        secondary["v2_gqa_8k"]["lam_logits_TFLOP/s"] = round(tf, 2)
        log(f"[bench]   lambda logits: {avg:.3f} ms -> {tf:.1f} TFLOP/s")
        del x5, o5, z5
    if "decode" in which:
        c4 = W.V1_DECODE_64K
        log(f"[bench] {c4.name} (generating the cache on the device)")
        x4 = W.decode_inputs(c4, device=dev)
        lam4 = x4["lam"].to(dev)
        ws = torch.empty(da.diffattn_decode_workspace_size(c4.B, c4.H, c4.L, c4.dv), dtype=torch.uint8, device=dev)
        o4 = torch.empty((c4.B, c4.H, c4.dv), dtype=torch.bfloat16, device=dev)
        f4 = lambda: da.diffattn_decode(x4["q1"], x4["q2"], x4["k1"], x4["k2"], x4["v"], lam4, epilogue=True,
                                        lambda_init_value=c4.lambda_init, workspace=ws, out=o4)
        f4()
        torch.cuda.synchronize()
        _r = measure(f4, torch, "v1_decode", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        nbytes = DECODE_BYTES_PER_TOKEN * c4.B * c4.H * c4.L
        gbs = nbytes / (avg * 1e-3) / 1e9
        secondary["v1_decode_64k"] = {"workload": c4.name, "split_plus_reduce_median_ms": round(avg, 4),
                                      "min_ms": round(mn, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                                      "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": load_traffic("v1_decode_64k", ["decode.hip", "common.hpp"])}
        log(f"[bench]   {avg:.3f} ms -> {gbs:.0f} GB/s")
        # the same cache in 256-token pages of a shared pool, in a random page order
        (p1, p2, pv), table = W.scatter_to_pages((x4["k1"], x4["k2"], x4["v"]), PAGE_SIZE, seed=c4.seed + 50)
        del x4["k1"], x4["k2"], x4["v"]
        fp = lambda: da.diffattn_decode_paged(x4["q1"], x4["q2"], p1, p2, pv, table, lam4, max_len=c4.L,
                                              epilogue=True, lambda_init_value=c4.lambda_init, workspace=ws, out=o4)
        fp()
        torch.cuda.synchronize()
        _r = measure(fp, torch, "v1_decode_paged", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        gbs = nbytes / (avg * 1e-3) / 1e9
        secondary["v1_decode_64k_paged"] = {"workload": c4.name + f", {PAGE_SIZE}-token pages",
                                            "split_plus_reduce_median_ms": round(avg, 4), "min_ms": round(mn, 4),
                                            "bytes": nbytes, "GB/s": round(gbs, 1),
                                            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench]   paged: {avg:.3f} ms -> {gbs:.0f} GB/s")
        del x4, ws, o4, p1, p2, pv, table
    if "bwd" in which:
        # training step of the main workload: the training forward and the backward pass
        c7 = W.V1_PREFILL_2K
        log(f"[bench] backward, {c7.name}")
        x7 = W.v1_inputs(c7, device=dev)
        lam7 = da.diffattn_lambda(*(x7[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), c7.layer)
        li7 = da.lambda_init(c7.layer)
        g7 = torch.Generator(device=dev).manual_seed(7)
        dy7 = torch.randn((c7.B, c7.N, c7.H, c7.dv), generator=g7, device=dev).to(torch.bfloat16)
        args7 = (x7["q1"], x7["q2"], x7["k1"], x7["k2"], x7["v"])
        ft = lambda: da.diffattn_fwd_train(*args7, lam7, causal=True, epilogue=True, lambda_init_value=li7)
        _, lse7, maps7 = ft()
        ws7 = torch.empty(da.diffattn_bwd_workspace_size(c7.B, c7.H, c7.N), dtype=torch.uint8, device=dev)
        fb = lambda: da.diffattn_bwd(*args7, dy7, lam7, lse7, maps7, causal=True, epilogue=True,
                                     lambda_init_value=li7, workspace=ws7)
        fb()
        torch.cuda.synchronize()
        _r = measure(ft, torch, "v1_train_forward", samples=args.secondary_samples)
        avg_f, mn_f = _r["median"], _r["min"]
        _r = measure(fb, torch, "v1_backward", samples=args.secondary_samples)
        avg_b, mn_b = _r["median"], _r["min"]
        pairs7 = c7.B * c7.H * causal_pairs(c7.N)
        fl_b = FLOP_PER_PAIR_V1_BWD * pairs7
        secondary["v1_backward_2k"] = {"workload": c7.name, "train_forward_median_ms": round(avg_f, 4),
                                       "backward_median_ms": round(avg_b, 4), "backward_min_ms": round(mn_b, 4),
                                       "flop": fl_b, "flop_per_visible_pair": FLOP_PER_PAIR_V1_BWD,
                                       "TFLOP/s": round(fl_b / (avg_b * 1e-3) / 1e12, 2),
                                       "frac_of_bf16_peak": round(fl_b / (avg_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench]   training forward {avg_f:.3f} ms, backward {avg_b:.3f} ms -> "
            f"{fl_b / (avg_b * 1e-3) / 1e12:.1f} TFLOP/s")
        del x7, dy7, lse7, maps7, ws7
    if "fp8" in which:
        # the main workload with the score operands in fp8 (e4m3, dynamic absmax per (batch, head))
        c9 = W.V1_PREFILL_2K
        log(f"[bench] fp8 score operands, {c9.name}")
        x9 = W.v1_inputs(c9, device=dev)
        lam9 = da.diffattn_lambda(*(x9[k].to(dev) for k in ("lq1", "lk1", "lq2", "lk2")), c9.layer)
        li9 = da.lambda_init(c9.layer)
        o9 = torch.empty((c9.B, c9.N, c9.H, c9.dv), dtype=torch.bfloat16, device=dev)
        codes9, sc9, am9 = da.diffattn_quantize_fp8_qk(x9["q1"], x9["q2"], x9["k1"], x9["k2"])
        # the quantiser's C-ABI arguments marshalled once (as for the main step): the kernel takes
        # about 20 us, less than the Python binding's own argument checks
        q_args = (*(da._t4(x9[k]) for k in ("q1", "q2", "k1", "k2")), c9.B, c9.N, c9.N, c9.H, c9.d,
                  *(da._t4(o) for o in codes9), sc9.data_ptr(), am9.data_ptr(), stream)
        fq9 = lambda: da._check(L.diffattn_quantize_fp8_qk(*q_args))
        ff9 = lambda: da.diffattn_fwd_fp8(*codes9, sc9[0], sc9[1], sc9[2], sc9[3], x9["v"], lam9, causal=True,
                                          epilogue=True, lambda_init_value=li9, out=o9)
        o9b = torch.empty_like(o9)
        fb9 = lambda: da.diffattn_fwd(x9["q1"], x9["q2"], x9["k1"], x9["k2"], x9["v"], lam9, causal=True,
                                      epilogue=True, lambda_init_value=li9, out=o9b)

        def fs9():
            fq9()
            ff9()
        fq9()
        ff9()
        torch.cuda.synchronize()
        _r = measure(fq9, torch, "fp8_quantize", samples=args.secondary_samples)
        avg_q = _r["median"]
        _r = measure(ff9, torch, "fp8_forward", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        avg_s = measure(fs9, torch, "fp8_quantize_plus_forward", samples=args.secondary_samples)["median"]
        avg_b = measure(fb9, torch, "bf16_forward", samples=args.secondary_samples)["median"]
        fl9 = FLOP_PER_PAIR_V1 * c9.B * c9.H * causal_pairs(c9.N)
        tf = fl9 / (avg * 1e-3) / 1e12
        secondary["v1_prefill_2k_fp8_logits"] = {
            "workload": c9.name + ", Q1 Q2 K1 K2 in fp8 e4m3", "kernel_median_ms": round(avg, 4),
            "kernel_min_ms": round(mn, 4), "flop": fl9, "TFLOP/s": round(tf, 2),
            "quantize_four_operands_median_ms": round(avg_q, 4),
            "quantize_plus_forward_median_ms": round(avg_s, 4),
            "bf16_forward_median_ms": round(avg_b, 4)}
        log(f"[bench]   {avg:.3f} ms -> {tf:.1f} TFLOP/s (quantising Q1, Q2, K1, K2: {avg_q:.3f} ms; "
            f"quantise + fp8 forward {avg_s:.3f} ms against bf16 forward {avg_b:.3f} ms)")
        del x9, o9, o9b, codes9, sc9
    if "v2bwd" in which:
        # training step of the V2 prefill workload: the V2 training forward and the V2 backward
        c8 = W.V2_GQA_8K
        log(f"[bench] V2 backward, {c8.name}")
        x8 = W.v2_inputs(c8, device=dev)
        g8 = torch.Generator(device=dev).manual_seed(9)
        dy8 = torch.randn((c8.B, c8.N, c8.hq // 2, c8.d), generator=g8, device=dev).to(torch.bfloat16)
        ft8 = lambda: da.diffattn_v2_fwd_train(x8["q"], x8["k"], x8["v"], x8["lam"], causal=True)
        _, lse8, maps8 = ft8()
        ws8 = torch.empty(da.diffattn_v2_bwd_workspace_size(c8.B, c8.hq // 2, c8.N), dtype=torch.uint8, device=dev)
        fb8 = lambda: da.diffattn_v2_bwd(x8["q"], x8["k"], x8["v"], dy8, x8["lam"], lse8, maps8, causal=True,
                                         workspace=ws8)
        fb8()
        torch.cuda.synchronize()
        _r = measure(ft8, torch, "v2_train_forward", samples=args.secondary_samples)
        avg_f, _ = _r["median"], _r["min"]
        _r = measure(fb8, torch, "v2_backward", samples=args.secondary_samples)
        avg_b, mn_b = _r["median"], _r["min"]
        fl8 = FLOP_PER_PAIR_V2_BWD * c8.B * c8.hq * causal_pairs(c8.N)
        secondary["v2_backward_8k"] = {"workload": c8.name, "train_forward_median_ms": round(avg_f, 4),
                                       "backward_median_ms": round(avg_b, 4), "backward_min_ms": round(mn_b, 4),
                                       "flop": fl8, "flop_per_visible_pair_and_query_head": FLOP_PER_PAIR_V2_BWD,
                                       "TFLOP/s": round(fl8 / (avg_b * 1e-3) / 1e12, 2),
                                       "frac_of_bf16_peak": round(fl8 / (avg_b * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench]   training forward {avg_f:.3f} ms, backward {avg_b:.3f} ms -> "
            f"{fl8 / (avg_b * 1e-3) / 1e12:.1f} TFLOP/s")
        del x8, dy8, lse8, maps8, ws8
    if "v2decode" in which:
        c6 = W.V2_DECODE_64K
        log(f"[bench] {c6.name} (generating the cache on the device)")
        x6 = W.v2_decode_inputs(c6, device=dev)
        lam6 = x6["lam"].to(dev)
        ws6 = torch.empty(da.diffattn_v2_decode_workspace_size(c6.B, c6.hq // 2, c6.hkv, c6.L), dtype=torch.uint8,
                          device=dev)
        o6 = torch.empty((c6.B, c6.hq // 2, c6.d), dtype=torch.bfloat16, device=dev)
        f6 = lambda: da.diffattn_v2_decode(x6["q"], x6["k"], x6["v"], lam6, workspace=ws6, out=o6)
        f6()
        torch.cuda.synchronize()
        _r = measure(f6, torch, "v2_decode", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        nbytes = 2 * c6.d * 2 * c6.B * c6.hkv * c6.L     # K and V rows read once per KV head
        gbs = nbytes / (avg * 1e-3) / 1e9
        secondary["v2_decode_64k"] = {"workload": c6.name, "split_plus_reduce_median_ms": round(avg, 4),
                                      "min_ms": round(mn, 4), "bytes": nbytes, "GB/s": round(gbs, 1),
                                      "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                                      "traffic": load_traffic("v2_decode_64k", ["decode_v2.hip", "mfma_tile.hpp",
                                                                                "common.hpp"])}
        log(f"[bench]   {avg:.3f} ms -> {gbs:.0f} GB/s")
        (pk6, pv6), table6 = W.scatter_to_pages((x6["k"], x6["v"]), PAGE_SIZE, seed=c6.seed + 50)
        del x6["k"], x6["v"]
        fp6 = lambda: da.diffattn_v2_decode_paged(x6["q"], pk6, pv6, table6, lam6, max_len=c6.L, workspace=ws6,
                                                  out=o6)
        fp6()
        torch.cuda.synchronize()
        _r = measure(fp6, torch, "v2_decode_paged", samples=args.secondary_samples)
        avg, mn = _r["median"], _r["min"]
        gbs = nbytes / (avg * 1e-3) / 1e9
        secondary["v2_decode_64k_paged"] = {"workload": c6.name + f", {PAGE_SIZE}-token pages",
                                            "split_plus_reduce_median_ms": round(avg, 4), "min_ms": round(mn, 4),
                                            "bytes": nbytes, "GB/s": round(gbs, 1),
                                            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
        log(f"[bench]   paged: {avg:.3f} ms -> {gbs:.0f} GB/s")
        del x6, ws6, o6, pk6, pv6, table6
    if secondary:
        result["secondary"] = secondary

    if args.copy_calibration:
        # a plain 1 GiB device-to-device copy: the reference kernel for HBM byte counters
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        # measured peaks beside the published ones: the copy's rate (bytes read + written) and
        # the dense bf16 MFMA probe of the library
        avg_c = time_launches(lambda: dst.copy_(src), torch, samples=10)["median"]
        copy_gbs = 2 * (1 << 30) / (avg_c * 1e-3) / 1e9
        del src, dst
        probe_out, probe_flop = da.diffattn_probe_mfma_peak(4096, 2000, device=dev)
        avg_p = time_launches(lambda: da.diffattn_probe_mfma_peak(4096, 2000, device=dev), torch, samples=5)["median"]
        mfma_tflops = probe_flop / (avg_p * 1e-3) / 1e12
        result["measured_peaks"] = {
            "hbm_torch_copy_GB/s": round(copy_gbs, 1), "mfma_bf16_TFLOP/s": round(mfma_tflops, 1),
            "how": "torch copy_ of 1 GiB on the device (bytes read + written; the decode kernels stream "
                   "faster than it) and diffattn_probe_mfma_peak (4096 blocks of 4 waves, 8 independent "
                   "v_mfma_f32_32x32x16_bf16 chains each)"}
        result["roofline"]["frac_of_measured_peak"] = round(result["roofline"]["achieved"] / mfma_tflops, 4)
        log(f"[bench] measured peaks: copy {copy_gbs:.0f} GB/s, bf16 MFMA {mfma_tflops:.0f} TFLOP/s")
        del probe_out

    # ---------------- CPU baseline: the fp64 oracle on a bounded sample ----------------
    if args.cpu_baseline:
        import oracle
        x = W.v1_inputs(cfg, device="cpu")
        host = {k: head_major_f64(x[k]) for k in ("q1", "q2", "k1", "k2", "v")}
        lam_ref = oracle.lam(*(x[k].double().numpy() for k in ("lq1", "lk1", "lq2", "lk2")), cfg.layer)
        units_done, t_cpu, pairs = 0, 0.0, 0
        for b in range(cfg.B):
            for h in range(cfg.H):
                rows = np.array([(b, h, i) for i in range(cfg.N)])
                s = time.perf_counter()
                oracle.v1_forward(host["q1"], host["q2"], host["k1"], host["k2"], host["v"], lam_ref,
                                  causal=True, epilogue=True,
                                  lambda_init_value=oracle.lambda_init(cfg.layer), rows=rows)
                t_cpu += time.perf_counter() - s
                units_done += 1
                pairs += causal_pairs(cfg.N)
                if t_cpu > 20.0:
                    break
            if t_cpu > 20.0:
                break
        cpu_tf = FLOP_PER_PAIR_V1 * pairs / t_cpu / 1e12
        del x, host
        cores = oracle.num_threads()
        result["cpu_baseline"] = {"value": round(cpu_tf, 6), "unit": "TFLOP/s", "cores": cores,
                                  "kind": "oracle", "cpu_model": cpu_model(),
                                  "sample": f"{units_done} of {cfg.B * cfg.H} (batch, head) units of the main "
                                            f"workload, every row ({pairs} visible pairs), fp64, "
                                            f"{t_cpu:.1f} s (capped at 20 s)"}
        log(f"[bench] oracle: {units_done} units in {t_cpu:.1f} s -> {cpu_tf * 1e3:.3f} GFLOP/s "
            f"on {cores} threads ({cpu_model()})")
        # the long-context and V2 workloads: a seeded row sample per head (or pair), timed, and the
        # full-size oracle time extrapolated linearly in visible pairs (labelled as such)
        others = {}
        rng = np.random.default_rng(12345)
        c3 = W.V1_PREFILL_32K
        x3 = W.v1_inputs(c3, device=dev)          # the inputs the GPU leg timed, copied to the host
        h3 = {k: head_major_f64(x3[k]) for k in ("q1", "q2", "k1", "k2", "v")}
        lam3 = oracle.lam(*(x3[k].double().numpy() for k in ("lq1", "lk1", "lq2", "lk2")), c3.layer)
        rows3 = sample_rows(c3.N, rng)
        sel = np.array([(0, h, i) for h in range(c3.H) for i in rows3])
        s = time.perf_counter()
        oracle.v1_forward(h3["q1"], h3["q2"], h3["k1"], h3["k2"], h3["v"], lam3, causal=True, epilogue=True,
                          lambda_init_value=oracle.lambda_init(c3.layer), rows=sel)
        t3 = time.perf_counter() - s
        p3 = c3.H * sum(i + 1 for i in rows3)
        full3 = c3.B * c3.H * causal_pairs(c3.N)
        others["v1_prefill_32k"] = {"workload": c3.name, "sample": f"{len(rows3)} rows per head x {c3.H} heads "
                                    f"(last row, tile-boundary rows, 48 seeded random rows; {p3} visible pairs)",
                                    "sample_s": round(t3, 3), "TFLOP/s": round(FLOP_PER_PAIR_V1 * p3 / t3 / 1e12, 6),
                                    "full_size_s_extrapolated": round(t3 * full3 / p3, 1)}
        del x3, h3
        c5 = W.V2_GQA_8K
        x5 = W.v2_inputs(c5, device=dev)
        h5 = {k: head_major_f64(x5[k]) for k in ("q", "k", "v")}
        rows5 = sample_rows(c5.N, rng)
        sel = np.array([(b, p, i) for b in range(c5.B) for p in range(c5.hq // 2) for i in rows5])
        s = time.perf_counter()
        oracle.v2_forward(h5["q"], h5["k"], h5["v"], x5["lam"].double().cpu().numpy(), causal=True, rows=sel)
        t5 = time.perf_counter() - s
        p5 = c5.B * (c5.hq // 2) * sum(i + 1 for i in rows5)       # visible pairs per pair of query heads
        full5 = c5.B * (c5.hq // 2) * causal_pairs(c5.N)
        others["v2_gqa_8k"] = {"workload": c5.name, "sample": f"{len(rows5)} rows per (batch, pair) x "
                               f"{c5.B * c5.hq // 2} (both query heads of each pair; {p5} visible pairs)",
                               "sample_s": round(t5, 3),
                               "TFLOP/s": round(2 * FLOP_PER_PAIR_V2 * p5 / t5 / 1e12, 6),
                               "full_size_s_extrapolated": round(t5 * full5 / p5, 1)}
        del x5, h5
        result["cpu_baseline"]["other_workloads"] = others
        log(f"[bench] oracle samples: 32K {t3:.2f} s (full size ~{t3 * full3 / p3:.0f} s extrapolated), "
            f"V2 8K {t5:.2f} s (~{t5 * full5 / p5:.0f} s)")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

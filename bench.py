"""Throughput of the Representation Shift hot path on one MI355X.

One step = one rs_encoder_forward over one batch of the DeiT-S-shaped workload
(256 images x 197 tokens, C 384, 6 heads, MLP 1536, 12 blocks, bf16, pruning after
blocks 3/6/9 keeping 70% of the current tokens, class token kept): every block's
LayerNorms, QKV GEMM, fused attention, projection, fc1+GELU, fc2 with the fused score,
and the three top-k + compaction stages.  Inputs and weights are synthetic (seeded,
N(0,1) inputs, N(0, 0.02^2) weights) and resident in HBM before timing starts.

Prints one JSON line.  Also measured inside the timed region: the dominant kernel's
summed HIP-event time (events recorded on the stream the kernel is launched on) and its
algorithmic work, giving the roofline fraction; and the fp64 CPU oracle on a bounded
sample of the same workload (cpu_baseline).

    python bench.py [--steps K] [--warmup W] [--workload deit_s] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "img/s (DeiT-S/B) & vid/s (UMT-B/L-shaped) w/ RS pruning, 1 GPU; % roofline"
PEAK = {"mfma": 2500.0, "hbm": 8000.0}   # bf16 dense TFLOP/s, HBM GB/s (MI355X published)
KERNEL_BOUND = {"qkv": "mfma", "attention": "mfma", "proj": "mfma", "fc1": "mfma",
                "fc2_score": "mfma", "layernorm": "hbm", "topk": "hbm", "gather": "hbm",
                "score": "hbm"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(wl, x, blocks, budget_s=12.0):
    """The fp64 oracle encoder on as many whole samples as fit a ~10-30 s budget."""
    import numpy as np
    from oracle import rs_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    n, t_total = 0, 0.0
    while n < wl.B:
        t0 = time.perf_counter()
        O.encoder_forward(x[n], blocks, wl.heads, wl.prune_layers, wl.keep_ratios, wl.has_cls,
                          wl.ln_eps)
        t_total += time.perf_counter() - t0
        n += 1
        if t_total >= budget_s:
            break
    return {"value": n / t_total, "unit": f"{wl.unit}/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{n} of {wl.B} {wl.unit}s of the same workload through the full "
                      f"{wl.depth}-block pruned encoder, fp64 NumPy, {t_total:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deit_s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--breakdown", action="store_true", help="also time every kernel class")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path shards by sample with no communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import vit_token_pruning_amd as rs

    wl = synth.WORKLOADS[args.workload]
    if wl.depth == 1:
        sys.exit("pick an encoder workload")
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    torch.cuda.set_device(0)
    x_np = synth.make_input(wl, 0)
    blocks_np = synth.make_encoder_weights(wl, 0)
    x = torch.from_numpy(x_np).cuda().to(dt)
    blocks = [{n: torch.from_numpy(v).cuda().to(dt) for n, v in w.items()} for w in blocks_np]
    spec = rs.ModelSpec(wl.C, wl.heads, wl.hidden, dt, wl.has_cls, wl.ln_eps)
    enc = rs.Encoder(spec, blocks, wl.B, wl.L, wl.prune_layers, wl.keep_ratios)
    log(f"workload {wl.name}: B={wl.B} L={wl.L} -> {enc.L_final}, C={wl.C}, depth={wl.depth}")

    for _ in range(args.warmup):
        enc.forward(x)
    torch.cuda.synchronize()

    # per-kernel breakdown (one step per kernel class) to find the dominant kernel
    per = {}
    for kname in rs.KERNELS:
        if kname == "score":
            continue
        with rs.KernelTimer(kname) as kt:
            enc.forward(x)
        per[kname] = {"ms": kt.total_ms, "launches": kt.launches, "work": kt.work}
    dominant = max(per, key=lambda k: per[k]["ms"])
    log("per-kernel ms/step:", {k: round(v["ms"], 4) for k, v in per.items()}, "dominant:", dominant)

    # timed region: K steps; the dominant kernel is event-timed on its launch stream
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with rs.KernelTimer(dominant) as kt:
        start.record(stream)
        for _ in range(args.steps):
            enc.forward(x)
        end.record(stream)
        torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    value = wl.B / (ms_step / 1e3)
    log(f"timed {args.steps} steps: {ms_step:.4f} ms/step, {value:.1f} {wl.unit}/s")

    bound = KERNEL_BOUND[dominant]
    if bound == "mfma":
        achieved = kt.work / (kt.total_ms / 1e3) / 1e12
        unit = "TFLOP/s"
    else:
        achieved = kt.work / (kt.total_ms / 1e3) / 1e9
        unit = "GB/s"
    roof = {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2), "peak": PEAK[bound],
            "unit": unit, "frac": round(achieved / PEAK[bound], 4), "traffic": None,
            "launches_per_step": kt.launches // args.steps,
            "avg_launch_us": round(kt.total_ms * 1e3 / max(1, kt.launches), 3)}

    # algorithmic flop of one step under the schedule: 2 * (12 L C^2 + 2 L^2 C) per sample-block
    from_sched = 0.0
    L = wl.L
    for b in range(wl.depth):
        from_sched += 2.0 * (12 * L * wl.C ** 2 + 2 * L * L * wl.C)
        if b in wl.prune_layers:
            L = int(np.floor(wl.keep_ratios[list(wl.prune_layers).index(b)] * L + 0.5))
    tflops = from_sched * wl.B / (ms_step / 1e3) / 1e12

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": f"{wl.unit}/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, N(0,0.02^2) weights)",
        "config": {"workload": f"{wl.name} encoder, RS pruning", "batch": wl.B, "tokens": wl.L,
                   "tokens_out": enc.L_final, "C": wl.C, "heads": wl.heads, "hidden": wl.hidden,
                   "depth": wl.depth, "prune_after_blocks": list(wl.prune_layers),
                   "keep_ratios": list(wl.keep_ratios), "has_cls": wl.has_cls},
        "tokens_per_s": round(value * wl.L, 1),
        "encoder_tflops": round(tflops, 2),
        "roofline": roof,
        "kernel_ms_per_step": {k: round(v["ms"], 4) for k, v in per.items()},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, x_np, blocks_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

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
PEAK = {"mfma": 2500.0, "hbm": 8000.0}
BREAKDOWN_STEPS = 5   # steps per kernel class in the single-lane breakdown (fc1 and fc2 are close)   # bf16 dense TFLOP/s, HBM GB/s (MI355X published)
KERNEL_BOUND = {"qkv": "mfma", "attention": "mfma", "proj": "mfma", "fc1": "mfma",
                "fc2_score": "mfma", "ln_prep": "hbm", "topk": "hbm",
                "score": "hbm", "patch_embed": "mfma", "head": "mfma"}


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


# device kernel symbol (mangled) -> kernel class of the library's timing interface
# The pages' throughput for their own settings ("Representation Shift: Unifying Token
# Compression with FlashAttention", Table 5 for DeiT at batch 512, Tables 2 and 4 for UMT at
# batch 20 x 12 frames), measured on an NVIDIA RTX A6000 over the whole forward pass
# (patch embedding and head included) -- context only, not the same work as the encoder
# timed here, so it is reported beside `vs_baseline` (which stays null).
PAGES_CONTEXT = {
    "deit_t512": (13296, "Table 5, DeiT-T, Ours"), "deit_s512": (5948, "Table 5, DeiT-S, Ours"),
    "deit_b512": (2428, "Table 5, DeiT-B, Ours"), "umt_b12f_ret": (175, "Table 2, UMT-B, Ours"),
    "umt_l12f_ret": (66, "Table 2, UMT-L, Ours"), "umt_b12f_qa": (128, "Table 4, UMT-B, Ours"),
    "umt_l12f_qa": (46, "Table 4, UMT-L, Ours"),
}


def kernel_class(mangled: str):
    import re
    # the GEMM and, when K is split, its reduction kernel (which runs the epilogue)
    m = re.search(r"(?:gemm_kernel|splitk_reduce_kernel)I(DF16b|f)Li(\d)E", mangled)
    if m:
        return {"0": "qkv", "1": "proj", "2": "fc1", "3": "fc2_score", "4": "patch_embed",
                "5": "head"}[m.group(2)]
    for key, name in (("attention_kernel", "attention"), ("row_stats_kernel", "ln_prep"), ("fold_kernel", "ln_prep"),
                      ("topk_kernel", "topk"), ("score_kernel", "score"),
                      ("cls_rows_kernel", "patch_embed"), ("pool_partial_kernel", "head"),
                      ("pool_finish_kernel", "head")):
        if key in mangled:
            return name
    return None


def copy_probe(rs, torch):
    """A plain copy of known size through rs_topk_gather (selection and copy in one launch):
    2 GiB of bf16 rows, all kept (k = L), so the launch reads and writes exactly 2 GiB (+ the
    512 KiB of scores and of indices).  At 8x the 256 MB Infinity Cache, at most ~1/8 of the
    source can be cache-resident."""
    B, L, C = 8, 16384, 8192
    x = torch.randn(B, L, C, device="cuda").to(torch.bfloat16)
    s = torch.ones(B, L, device="cuda", dtype=torch.float32)
    for _ in range(3):
        rs.topk_gather(s, x, L, False)
    torch.cuda.synchronize()
    return B * L * C * 2


def summarize(dirs, workload):
    """Per-kernel averages of the counters (and dispatch durations) in rocprofv3 result
    databases; HBM traffic of each kernel class from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), scaled by what the same counters read for the 2 GiB copy probe (a top-k
    dispatch of over 100 us: the encoder's take tens); matrix-core busy fraction from
    SQ_VALU_MFMA_BUSY_CYCLES (summed over all SIMDs) against 1024 SIMDs x the dispatch
    duration at 2.4 GHz, also per launch shape ("by_grid": dispatches grouped by their grid
    size in work-items, which tells the prune stages apart)."""
    import collections
    import glob
    import sqlite3
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    by_grid = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(list)))
    probe = collections.defaultdict(list)
    for d in dirs:
        for path in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            cur = sqlite3.connect(path).cursor()
            names = dict(cur.execute("select id, kernel_name from kernel_symbols"))
            disp = {r[0]: (r[1], r[2]) for r in cur.execute(
                "select dispatch_id, kernel_id, duration from kernels")}
            grids = {r[0]: r[1] * r[2] * r[3] for r in cur.execute(
                "select dispatch_id, grid_x, grid_y, grid_z from kernels")}
            durs = collections.defaultdict(list)
            per_disp = collections.defaultdict(dict)
            for kid, dur in disp.values():
                kc = kernel_class(names.get(kid, ""))
                if kc is not None:
                    durs[kc].append(dur)
            has_sq = False
            for did, cname, cval in cur.execute(
                    "select dispatch_id, counter_name, sum(counter_value) from pmc_events "
                    "group by dispatch_id, counter_name"):
                has_sq = has_sq or cname.startswith("SQ_")
                kid, dur = disp.get(did, (None, 0))
                kc = kernel_class(names.get(kid, ""))
                if kc is None:
                    continue
                if kc == "topk" and dur > 100e3:
                    probe[cname].append(cval)
                else:
                    vals[kc][cname].append(cval)
                    per_disp[did][cname] = cval
            if has_sq:   # durations of the run whose counters give the busy fractions
                for kc, v in durs.items():
                    vals[kc]["duration_ns"].extend(d for d in v if not (kc == "topk" and d > 100e3))
                for did, cs in per_disp.items():
                    kid, dur = disp[did]
                    g = by_grid[kernel_class(names.get(kid, ""))][grids[did]]
                    g["duration_ns"].append(dur)
                    for cname, cval in cs.items():
                        g[cname].append(cval)
    known = 8 * 16384 * 8192 * 2
    out = {"workload": workload, "kernels": {}}
    fac = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        if probe.get(c):
            fac[c] = known / (sum(probe[c]) / len(probe[c]) * 1024.0)
    out["copy_probe"] = {"bytes_each_way": known,
                         **{c: sum(v) / len(v) for c, v in probe.items()}, "scale": fac}
    for kc, cs in vals.items():
        row = {c: sum(v) / len(v) for c, v in cs.items()}
        row["dispatches"] = max(len(v) for v in cs.values())
        t = 0.0
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in row and c in fac:
                row[c + "_bytes"] = row[c] * 1024.0 * fac[c]
                t += row[c + "_bytes"]
        if "FETCH_SIZE_bytes" in row and "WRITE_SIZE_bytes" in row:
            row["traffic_bytes_per_launch"] = t
        if "SQ_VALU_MFMA_BUSY_CYCLES" in row and row.get("duration_ns"):
            row["mfma_busy_frac"] = row["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * row["duration_ns"] * 2.4)
        if kc in by_grid:
            row["by_grid"] = {}
            for grid, gs in sorted(by_grid[kc].items(), reverse=True):
                g = {c: sum(v) / len(v) for c, v in gs.items()}
                g["dispatches"] = len(gs["duration_ns"])
                if "SQ_VALU_MFMA_BUSY_CYCLES" in g and g["duration_ns"]:
                    g["mfma_busy_frac"] = g["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * g["duration_ns"] * 2.4)
                row["by_grid"][str(grid)] = g
        out["kernels"][kc] = row
    out["kernel_sources_sha256"] = kernel_sources_sha256()
    return out


def kernel_sources_sha256():
    import hashlib
    src = os.path.join(ROOT, "vit_token_pruning_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            h.update(open(os.path.join(src, f), "rb").read())
    return h.hexdigest()


def stored_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from profiles/traffic_<workload>.json, only if the
    counters were taken on the kernel sources as they are now."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    k = t.get("kernels", {}).get(kernel, {})
    v = k.get("traffic_bytes_per_launch")
    return None if v is None else float(v)


def standalone(wl, steps):
    """rs_score and rs_topk_gather alone at the workload's prune-stage shapes: algorithmic
    bytes / kernel time against 8 TB/s.  Inputs rotate over >= 512 MiB of buffers (twice the
    256 MB Infinity Cache) so every call reads from HBM.  Bytes per call: rs_score reads
    f and x (2 M C e) and writes 4 M; rs_topk_gather reads 4 L scores and the k kept rows
    (k C e) per sample and writes k C e + 4 k."""
    import numpy as np
    import torch
    from vit_token_pruning_amd import _native as N
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    e = 2 if wl.dtype == "bf16" else 4
    lib = N.lib()
    code = N.RS_BF16 if wl.dtype == "bf16" else N.RS_F32
    stream = torch.cuda.current_stream()
    out = []
    L = wl.L
    for pl, r in zip(wl.prune_layers, wl.keep_ratios):
        k = int(np.floor(r * L + 0.5))
        B, C = wl.B, wl.C
        M = B * L
        nbuf = max(2, -(-(512 << 20) // (2 * M * C * e)))
        g = torch.Generator(device="cuda").manual_seed(0)
        fx = [torch.randn(B, L, C, device="cuda", generator=g).to(dt) for _ in range(nbuf)]
        xs = [torch.randn(B, L, C, device="cuda", generator=g).to(dt) for _ in range(nbuf)]
        sc = [torch.empty(B, L, device="cuda", dtype=torch.float32) for _ in range(nbuf)]
        kept = torch.empty(B, k, device="cuda", dtype=torch.int32)
        xk = torch.empty(B, k, C, device="cuda", dtype=dt)
        hs = stream.cuda_stream

        def score(i):
            N.check("rs_score", lib.rs_score(fx[i].data_ptr(), xs[i].data_ptr(), B, L, C, code,
                                             sc[i].data_ptr(), hs))

        def select(i):
            N.check("rs_topk_gather", lib.rs_topk_gather(sc[i].data_ptr(), xs[i].data_ptr(), B, L, C,
                                                         code, k, wl.has_cls, kept.data_ptr(),
                                                         xk.data_ptr(), hs))
        for i in range(nbuf):
            score(i)
        torch.cuda.synchronize()
        res = {"after_block": pl, "L": L, "k": k, "M": M, "buffers_MiB": round(nbuf * 2 * M * C * e / 2**20)}
        for name, fn, nbytes in (("score", score, 2.0 * M * C * e + 4.0 * M),
                                 ("topk_gather", select, B * (4.0 * L + 2.0 * k * C * e + 4.0 * k))):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for it in range(steps):
                fn(it % nbuf)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            gbs = nbytes / (us * 1e-6) / 1e9
            res[name] = {"us": round(us, 2), "bytes": int(nbytes), "GB_s": round(gbs, 1),
                         "frac_hbm": round(gbs / PEAK["hbm"], 4)}
        out.append(res)
        del fx, xs, sc
        torch.cuda.empty_cache()
        L = k
    return out


def compare(wl, blocks, x, steps, ours, rs, torch):
    """Context, not `value`: the pages' Base / Attn / Ours structure (Tables 2, 4, 5) on this
    GPU, encoder only, same weights and input.  base: no pruning, every attention forms and
    stores its map (a non-fused attention's output); base_fused: no pruning, fused
    attention; attn: stored maps and pruning by the attention-map score (Eq. (2) with a
    class token, else Eq. (3)) on the same schedule; ours: the method (the line's value)."""
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    op = "map_cls" if wl.has_cls else "map_mean"
    cfgs = {"base": ("mlp", True, (), ()), "base_fused": ("mlp", False, (), ()),
            "attn": (op, True, wl.prune_layers, wl.keep_ratios)}
    out = {}
    n = max(5, min(steps, 20))
    for name, (sop, amap, pl, kr) in cfgs.items():
        spec = rs.ModelSpec(wl.C, wl.heads, wl.hidden, dt, wl.has_cls, wl.ln_eps, score_op=sop,
                            attn_map=amap)
        enc = rs.Encoder(spec, blocks, wl.B, wl.L, pl, kr)
        for _ in range(3):
            enc.forward(x)
        stream = torch.cuda.current_stream()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(n):
            enc.forward(x)
        end.record(stream)
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / n
        out[name] = {"value": round(wl.B / (ms / 1e3), 2), "ms_per_step": round(ms, 4)}
        del enc
        torch.cuda.empty_cache()
    out["ours"] = {"value": round(ours, 2)}
    out["attn_score"] = op
    out["ours_vs_attn"] = round(ours / out["attn"]["value"], 3)
    out["ours_vs_base"] = round(ours / out["base"]["value"], 3)
    log("comparison (encoder):", out)
    return out


def whole_forward(wl, spec, blocks, steps, rs, torch):
    """Context, not `value`: the whole forward pass (patch embedding, the same pruned
    encoder, final LayerNorm and head) from pixels resident in HBM, as the pages'
    throughput figures count it.  Synthetic 224 x 224 pixels, 16 x 16 patches."""
    import synth
    dt = spec.dtype
    g = synth.geometry(wl)
    img = rs.ImageSpec(g.frames, g.in_chans, g.height, g.width, g.patch)
    dev = lambda a: torch.from_numpy(a).cuda().to(dt)
    images = dev(synth.make_images(wl, g, 0))
    emb = {k: dev(v) for k, v in synth.make_embed_weights(wl, g, 0).items()}
    hw = {k: dev(v) for k, v in synth.make_head_weights(wl, g, 0).items()}
    vit = rs.ViT(spec, img, emb, blocks, hw, g.pool, wl.B, wl.prune_layers, wl.keep_ratios)
    for _ in range(3):
        vit.forward(images)
    n = max(5, min(steps, 20))
    stream = torch.cuda.current_stream()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(n):
        vit.forward(images)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / n
    per = {}
    for kname in ("patch_embed", "head"):
        with rs.KernelTimer(kname) as kt:
            vit.forward(images)
        per[kname] = {"ms": round(kt.total_ms, 4), "launches": kt.launches,
                      "tflops": round(kt.work / (kt.total_ms / 1e3) / 1e12, 1) if kt.total_ms else None}
    torch.cuda.synchronize()
    value = wl.B / (ms / 1e3)
    log(f"whole forward ({g.frames} x {g.height}x{g.width} px, patch {g.patch}, head {g.n_out}, "
        f"{g.pool} pool): {ms:.4f} ms/step, {value:.1f} {wl.unit}/s; {per}")
    return {"value": round(value, 2), "unit": f"{wl.unit}/s", "ms_per_step": round(ms, 4),
            "steps": n, "frames": g.frames, "pixels": [g.height, g.width], "patch": g.patch,
            "n_out": g.n_out, "pool": g.pool, "kernels": per,
            "note": "patch embedding + the pruned encoder + final LN + head; context only"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="deit_s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--standalone", action="store_true",
                    help="time rs_score and rs_topk_gather alone at the prune-stage shapes "
                         "(HBM-bound kernels, rotating >= 512 MiB of inputs); prints one JSON line")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the single-lane per-kernel breakdown and context pass, so every "
                         "launch in the process is a timed-mode launch (for profiler runs)")
    ap.add_argument("--kernel", default="fc2_score", choices=[k for k in ("ln_prep", "qkv", "attention",
                    "proj", "fc1", "fc2_score", "topk")],
                    help="roofline kernel when --no-breakdown is given")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the Base / Attn / Ours comparison (context)")
    ap.add_argument("--no-whole", action="store_true",
                    help="skip the whole-forward context (patch embedding + encoder + head)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 256 MiB copy through the gather kernel (counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="summarize rocprofv3 --pmc result directories and exit (no GPU use)")
    args = ap.parse_args()
    if args.summarize:
        print(json.dumps(summarize(args.summarize, args.workload), indent=1))
        return
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
    if args.standalone:
        torch.cuda.set_device(0)
        res = standalone(wl, args.steps)
        print(json.dumps({"metric": "standalone rs_score / rs_topk_gather HBM throughput",
                          "workload": wl.name, "unit": "GB/s", "peak": PEAK["hbm"], "stages": res}),
              flush=True)
        return
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

    def rate(work, ms):
        return work / (ms / 1e3) / (1e12 if bound == "mfma" else 1e9)

    # per-kernel breakdown (BREAKDOWN_STEPS steps per kernel class, averaged; single lane so
    # launches do not overlap) to find the dominant kernel
    per, kt1 = {}, None
    if args.no_breakdown:
        dominant = args.kernel
    else:
        rs.set_max_lanes(1)
        for kname in rs.KERNELS:
            if kname in ("score", "gather", "patch_embed", "head"):   # not launched by the encoder
                continue
            with rs.KernelTimer(kname) as kt:
                for _ in range(BREAKDOWN_STEPS):
                    enc.forward(x)
            per[kname] = {"ms": kt.total_ms / BREAKDOWN_STEPS, "launches": kt.launches // BREAKDOWN_STEPS,
                          "work": kt.work / BREAKDOWN_STEPS}
        dominant = max(per, key=lambda k: per[k]["ms"])
        log("per-kernel ms/step (single lane):", {k: round(v["ms"], 4) for k, v in per.items()},
            "dominant:", dominant)
        # the dominant kernel alone on the GPU: its unshared rate, for context
        with rs.KernelTimer(dominant) as kt1:
            for _ in range(min(args.steps, 10)):
                enc.forward(x)
        rs.set_max_lanes(2)
        torch.cuda.synchronize()
    bound = KERNEL_BOUND[dominant]

    # timed region: K steps of the encoder as it runs by default (two lanes when the batch
    # is large enough); the dominant kernel is event-timed on the stream each launch runs on
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

    achieved = rate(kt.work, kt.total_ms)
    roof = {"bound": bound, "kernel": dominant, "achieved": round(achieved, 2), "peak": PEAK[bound],
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s", "frac": round(achieved / PEAK[bound], 4),
            "traffic": stored_traffic(wl.name, dominant),
            "launches_per_step": kt.launches // args.steps,
            "avg_launch_us": round(kt.total_ms * 1e3 / max(1, kt.launches), 3),
            }
    if kt1 is not None:
        # launches of the two encoder lanes overlap in the timed region; the same kernel
        # with the batch on one stream (not timed for `value`):
        achieved1 = rate(kt1.work, kt1.total_ms)
        roof["single_lane"] = {"achieved": round(achieved1, 2), "frac": round(achieved1 / PEAK[bound], 4),
                               "avg_launch_us": round(kt1.total_ms * 1e3 / max(1, kt1.launches), 3)}

    # algorithmic flop of one step under the schedule: 2 * (12 L C^2 + 2 L^2 C) per sample-block
    # and the token-blocks one sample passes through (tokens entering each block)
    from_sched, token_blocks = 0.0, 0
    L = wl.L
    for b in range(wl.depth):
        from_sched += 2.0 * (12 * L * wl.C ** 2 + 2 * L * L * wl.C)
        token_blocks += L
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
        "token_blocks_per_s": round(value * token_blocks, 1),
        "encoder_tflops": round(tflops, 2),
        "roofline": roof,
        "kernel_ms_per_step": {k: round(v["ms"], 4) for k, v in per.items()},  # single lane
    }
    if wl.name in PAGES_CONTEXT:
        v, cite = PAGES_CONTEXT[wl.name]
        line["pages_context"] = {"value": v, "unit": f"{wl.unit}/s", "source": cite,
                                 "note": "RTX A6000, whole forward pass; not the same work",
                                 "ratio": round(value / v, 2)}
    if not (args.no_compare or args.no_breakdown):
        line["comparison"] = compare(wl, blocks, x, args.steps, value, rs, torch)
    if not (args.no_whole or args.no_breakdown):
        line["whole_forward"] = whole_forward(wl, spec, blocks, args.steps, rs, torch)
        if wl.name in PAGES_CONTEXT:
            line["pages_context"]["ratio_whole_forward"] = round(
                line["whole_forward"]["value"] / PAGES_CONTEXT[wl.name][0], 2)
    if args.copy_probe:
        copy_probe(rs, torch)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, x_np, blocks_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

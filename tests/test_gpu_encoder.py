"""Full-size encoder parity (the four encoder workloads at their real batch and length,
the launch configuration the benchmark times).

rs_encoder_forward is checked bit-exactly against chains of rs_block_forward calls at
the same shapes (same kernels, deterministic), whose per-block results are checked
against the oracle on sampled samples with teacher forcing: the oracle block is fed the
GPU's own block input, so each comparison measures one block's rounding.  The encoder
runs a batch as n lanes (contiguous shares of the samples on n streams; n up to the
process-wide maximum, default 2) when every lane keeps >= 512 rows after the last
pruning; the reference chains run per lane, since a GEMM's split over K depends on its
row count and so on the lane's batch."""
import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, spec_of, to_dev,
                         to_host, weights_to_dev)

pytestmark = pytest.mark.gpu

SAMPLED = {"deit_s": [0, 255], "deit_b": [0, 127], "umt_b": [5], "umt_l": [2],
           "deit_s512": [511], "umt_l12f_ret": [13], "deit_t512": [0, 300], "deit_b512": [400],
           "umt_b12f_qa": [19], "umt_b12f_ret": [3], "umt_l12f_qa": [7]}


def lanes(B, L_final, max_lanes=2):
    n = max_lanes
    while n > 1 and (B < n or (B // n) * L_final < 512):
        n -= 1
    out, b0 = [], 0
    for i in range(n):
        b1 = b0 + B // n + (1 if i < B % n else 0)
        out.append((b0, b1))
        b0 = b1
    return out


def chain_and_check(wl, blocks, wd, xd, samp):
    """rs_block_forward chained over the encoder's schedule for the samples of xd, with
    teacher-forced oracle checks of every block on the sample indices `samp` (local to
    xd).  Returns the final rows, their original ids and the kept-set agreement count."""
    import torch
    import vit_token_pruning_amd as rs
    spec = spec_of(wl)
    _, ks, _ = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)
    cur = xd
    ids = np.tile(np.arange(wl.L), (xd.shape[0], 1))
    exact = total = 0
    for b in range(wl.depth):
        L = cur.shape[1]
        k = ks.get(b, L)
        cur_host = to_host(cur[samp]) if samp else None
        r = rs.block_forward(spec, wd[b], cur, k)
        torch.cuda.synchronize()
        kept_all = r["kept_idx"].cpu().numpy()
        if samp:
            y = to_host(r["y"][samp])
            s = r["scores"][samp].cpu().numpy()
        for j, sb in enumerate(samp):
            ora = O.block_forward(cur_host[j], blocks[b], wl.heads, wl.ln_eps)
            check_block_output(y[j], ora["x_hat"], cur_host[j], wl.dtype)
            check_scores(s[j], ora["score"])
            if b in ks:
                exact += kept_admissible(kept_all[sb], ora["score"], k, wl.has_cls)
                total += 1
        if b in ks:
            ids = np.take_along_axis(ids, kept_all.astype(np.int64), axis=1)
        cur = r["y_kept"]
    torch.cuda.synchronize()
    return cur, ids, exact, total


def check_encoder(wl, samples, max_lanes=2):
    import torch
    import vit_token_pruning_amd as rs
    spec = spec_of(wl)
    x = synth.make_input(wl, 0)
    blocks = synth.make_encoder_weights(wl, 0)
    wd = [weights_to_dev(w, wl.dtype) for w in blocks]
    xd = to_dev(x, wl.dtype)
    _, _, L_final = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)

    out, out_idx = rs.encoder_forward(spec, wd, xd, wl.prune_layers, wl.keep_ratios)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (wl.B, L_final, wl.C)

    exact = total = 0
    for b0, b1 in lanes(wl.B, L_final, max_lanes):
        samp = [s - b0 for s in samples if b0 <= s < b1]
        cur, ids, e, t = chain_and_check(wl, blocks, wd, xd[b0:b1].contiguous(), samp)
        exact, total = exact + e, total + t
        assert torch.equal(out[b0:b1], cur), f"encoder lane {b0}:{b1} differs from the chained blocks"
        assert np.array_equal(out_idx[b0:b1].cpu().numpy(), ids)
    print(f"{wl.name} B{wl.B}: exact kept-set agreement {exact}/{total} sampled prune stages")


@pytest.mark.parametrize("name", ["deit_s", "deit_b", "umt_b", "umt_l", "deit_s512", "umt_l12f_ret",
                                  "deit_t512", "deit_b512", "umt_b12f_qa", "umt_b12f_ret",
                                  "umt_l12f_qa"])
def test_encoder_full_size(name):
    check_encoder(synth.WORKLOADS[name], SAMPLED[name])


def test_encoder_full_size_ragged_rows():
    """DeiT-S at its full length and depth with 250 samples: lanes of 125 samples, so every
    stage's rows (125 x 197, x 138, x 97, x 68) end in a partial 128-row block of the
    weight-streaming QKV / projection kernel and the fused MLP."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=250)
    check_encoder(wl, [0, 249])


@pytest.mark.parametrize("B", [1, 3, 45])
def test_encoder_one_lane_and_uneven_lanes(B):
    """B = 1 and 3 run on the caller's stream alone (too few rows for two lanes); B = 45
    (48 tokens left) splits into lanes of 23 and 22 samples."""
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=B, L=97, depth=4, prune_layers=(1, 2),
                             keep_ratios=(0.7, 0.7))
    check_encoder(wl, [B - 1])


def test_encoder_lanes_setting():
    """rs_set_max_lanes(1) runs the whole batch on the caller's stream; with two lanes the
    results equal the per-lane chains (checked above), with one the full-batch chain."""
    import torch
    import vit_token_pruning_amd as rs
    import dataclasses
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=45, L=97, depth=3, prune_layers=(1,),
                             keep_ratios=(0.7,))
    spec = spec_of(wl)
    blocks = synth.make_encoder_weights(wl, 0)
    wd = [weights_to_dev(w, wl.dtype) for w in blocks]
    xd = to_dev(synth.make_input(wl, 0), wl.dtype)
    try:
        rs.set_max_lanes(1)
        out1, idx1 = rs.encoder_forward(spec, wd, xd, wl.prune_layers, wl.keep_ratios)
        torch.cuda.synchronize()
    finally:
        rs.set_max_lanes(2)
    cur, ids, _, _ = chain_and_check(wl, blocks, wd, xd, [])
    assert torch.equal(out1, cur)
    assert np.array_equal(idx1.cpu().numpy(), ids)


@pytest.mark.parametrize("B", [45, 3])
def test_encoder_replays_from_a_hip_graph(B):
    """The encoder (two lanes at B = 45, forked from and joined to the caller's stream
    with events; one lane at B = 3) can be captured in a HIP graph: every replay, with
    eager launches of the library and synchronisations in between, equals the eager run
    bit for bit.  The library allocates nothing and clears nothing with memset nodes."""
    import dataclasses
    import torch
    import vit_token_pruning_amd as rs
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=B, L=97, depth=3, prune_layers=(1,),
                             keep_ratios=(0.7,))
    spec = spec_of(wl)
    wd = [weights_to_dev(w, wl.dtype) for w in synth.make_encoder_weights(wl, 0)]
    xd = to_dev(synth.make_input(wl, 0), wl.dtype)
    enc = rs.Encoder(spec, wd, wl.B, wl.L, wl.prune_layers, wl.keep_ratios)
    out, idx = enc.forward(xd)
    torch.cuda.synchronize()
    ref, ref_idx = out.clone(), idx.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        enc.forward(xd)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        enc.forward(xd)
    torch.cuda.synchronize()
    other = rs.Encoder(spec, wd, wl.B, wl.L, wl.prune_layers, wl.keep_ratios)
    for _ in range(3):
        enc.out.zero_()
        enc.out_idx.zero_()
        other.forward(torch.flip(xd, dims=[1]).contiguous())   # eager work in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(enc.out, ref) and torch.equal(enc.out_idx, ref_idx)


@pytest.mark.parametrize("n", [3, 4])
def test_encoder_more_lanes(n):
    """rs_set_max_lanes(3 / 4): 64 samples keeping 68 tokens run as 3 lanes (22, 21, 21
    samples) or 4 lanes (16 each), each equal to its chain of blocks."""
    import dataclasses
    import vit_token_pruning_amd as rs
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=64, L=97, depth=3, prune_layers=(1,),
                             keep_ratios=(0.7,))
    try:
        rs.set_max_lanes(n)
        check_encoder(wl, [0, 63], max_lanes=n)
    finally:
        rs.set_max_lanes(2)


def test_encoder_concurrent_calls_on_two_streams():
    """Two host threads, each with its own stream and workspace, run the encoder at the same
    time (two lanes each, so both calls also fork onto the library's lane stream); every
    result equals the single-threaded run of the same input bit for bit."""
    import dataclasses
    import threading
    import torch
    import vit_token_pruning_amd as rs
    wl = dataclasses.replace(synth.WORKLOADS["deit_s"], B=45, L=97, depth=3, prune_layers=(1,),
                             keep_ratios=(0.7,))
    spec = spec_of(wl)
    wd = [weights_to_dev(w, wl.dtype) for w in synth.make_encoder_weights(wl, 0)]
    xs = [to_dev(synth.make_input(wl, seed), wl.dtype) for seed in (0, 1)]
    refs = []
    for x in xs:
        out, idx = rs.Encoder(spec, wd, wl.B, wl.L, wl.prune_layers, wl.keep_ratios).forward(x)
        torch.cuda.synchronize()
        refs.append((out.clone(), idx.clone()))
    encs = [rs.Encoder(spec, wd, wl.B, wl.L, wl.prune_layers, wl.keep_ratios) for _ in xs]
    streams = [torch.cuda.Stream() for _ in xs]
    torch.cuda.synchronize()
    results, errors = [[], []], []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for _ in range(4):
                    out, idx = encs[i].forward(xs[i])
                    results[i].append((out.clone(), idx.clone()))
            streams[i].synchronize()
        except Exception as e:  # reported below, on the main thread
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(xs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    for i, (ref_out, ref_idx) in enumerate(refs):
        assert len(results[i]) == 4
        for out, idx in results[i]:
            assert torch.equal(out, ref_out) and torch.equal(idx, ref_idx), f"thread {i}"

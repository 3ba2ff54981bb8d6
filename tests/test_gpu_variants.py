"""GPU parity of the score variants of the ablations ("Representation Shift", Sec. 3.3,
"Operation choice" and "Distance metrics"): the shift through the attention sublayer,
the MLP sublayer (the method) or the whole block, with the L2, L1 or cosine distance,
against the fp64 oracle.  The block output does not depend on the variant (checked
bit-exactly against the method's run); the standalone rs_score_dist is checked against
the oracle's distances and their closed forms; an encoder run with a variant equals the
chain of its blocks."""
import dataclasses

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, oracle_block,
                         spec_of, to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
VARIANTS = [(op, dist) for op in O.SHIFT_OPS for dist in O.DISTANCES]
# (workload, batch, stage length, keep ratio): one tile row and a ragged tail (DeiT-T),
# several tiles (DeiT-S), fp32 with K split in fc2 (DeiT-S) or in all four GEMMs (UMT-L),
# and the widest layer in bf16 (UMT-L)
SHAPES = [("deit_t_block", 2, 197, 0.7), ("deit_s", 3, 138, 0.7), ("deit_s@f32", 2, 97, 0.7),
          ("umt_l", 1, 392, 0.5), ("umt_l@f32", 1, 98, 0.5)]


def _wl(name):
    base, _, dt = name.partition("@")
    return dataclasses.replace(W[base], dtype=dt) if dt else W[base]


def _run(wl, op, dist, x, w, k):
    import torch
    import vit_token_pruning_amd as rs
    r = rs.block_forward(spec_of(wl, op, dist), weights_to_dev(w, wl.dtype), to_dev(x, wl.dtype), k)
    torch.cuda.synchronize()
    return r


@pytest.mark.parametrize("name,B,L,ratio", SHAPES)
@pytest.mark.parametrize("op,dist", VARIANTS)
def test_block_variant_matches_oracle(name, B, L, ratio, op, dist):
    wl = _wl(name)
    k = O.keep_count(ratio, L)
    x = synth.make_input(wl, 21 + L, B=B, L=L)
    w = synth.make_block_weights(wl, 0, 21 + L, init="full")
    r = _run(wl, op, dist, x, w, k)
    y, s = to_host(r["y"]), r["scores"].cpu().numpy()
    kept, yk = r["kept_idx"].cpu().numpy(), to_host(r["y_kept"])
    ora = oracle_block(x, w, wl.heads, wl.ln_eps, op=op, dist=dist)
    check_block_output(y, ora["x_hat"], x, wl.dtype)
    err = check_scores(s, ora["score"])
    exact = 0
    for b in range(B):
        exact += kept_admissible(kept[b], ora["score"][b], k, wl.has_cls)
        assert kept[b].tolist() == O.select_kept(s[b], k, wl.has_cls)
        np.testing.assert_array_equal(yk[b], y[b][kept[b]])
    # the variant changes the score only: the block output equals the method's bit for bit
    if (op, dist) != ("mlp", "l2"):
        assert np.array_equal(to_host(_run(wl, "mlp", "l2", x, w, k)["y"]), y)
    print(f"{name} B{B} L{L} {op}/{dist}: score rel err {err:.2e}, exact kept sets {exact}/{B}")


@pytest.mark.parametrize("name,L", [("deit_t_block", 197), ("umt_l@f32", 98)])
def test_variant_closed_forms(name, L):
    """Zero branches fix the variants' scores: with both branches zero x_hat = x, so the
    whole-block shift is 0 under every distance (all tokens tie: the lowest indices are
    kept); with the attention branch zero its shift is ||x||_2, sum |x| and cosine 1."""
    wl = _wl(name)
    B, k = 2, O.keep_count(0.5, L)
    x = synth.make_input(wl, 7, B=B, L=L)
    xd = x.astype(np.float64)
    w = synth.make_block_weights(wl, 0, 7, init="full", zero=("w_proj", "b_proj", "w_fc2", "b_fc2"))
    for dist in O.DISTANCES:
        r = _run(wl, "block", dist, x, w, k)
        s = r["scores"].cpu().numpy()
        assert np.abs(s).max() <= (0.0 if dist != "cos" else 1e-6), (dist, np.abs(s).max())
        if dist != "cos":
            want = list(range(k))
            assert all(r["kept_idx"][b].cpu().tolist() == want for b in range(B))
    w = synth.make_block_weights(wl, 0, 8, init="full", zero=("w_proj", "b_proj"))
    want = {"l2": np.linalg.norm(xd, axis=-1), "l1": np.abs(xd).sum(-1), "cos": np.ones((B, L))}
    for dist in O.DISTANCES:
        s = _run(wl, "attn", dist, x, w, k)["scores"].cpu().numpy()
        assert (np.abs(s - want[dist]) / want[dist]).max() <= 1e-5, dist


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("C", [64, 384, 1024, 1032])
def test_score_dist_matches_oracle(dt, C):
    import torch
    import vit_token_pruning_amd as rs
    rng = np.random.default_rng(C)
    B, L = 3, 37
    fx = rng.standard_normal((B, L, C)).astype(np.float32)
    x = rng.standard_normal((B, L, C)).astype(np.float32)
    fx[0, 0] = x[0, 0]            # identical rows: distance 0
    fx[0, 1] = 0.0                # zero row: cosine distance exactly 1
    fx[0, 2] = -x[0, 2]           # opposite rows: cosine distance 2
    fd, xd = to_dev(fx, dt), to_dev(x, dt)
    a, b = to_host(fd).astype(np.float64), to_host(xd).astype(np.float64)
    for dist in O.DISTANCES:
        s = rs.score(fd, xd, dist).cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
        want = O.representation_shift(a, b, dist)
        nz = np.abs(want) > 1e-3
        assert (np.abs(s - want)[nz] / want[nz]).max() <= 1e-5, dist
        assert np.abs(s - want)[~nz].max(initial=0.0) <= 1e-5, dist
        if dist != "cos":
            assert s[0, 0] == 0.0
        else:
            assert s[0, 1] == 1.0 and abs(s[0, 2] - 2.0) <= 1e-6
    assert np.array_equal(rs.score(fd, xd).cpu().numpy(), rs.score(fd, xd, "l2").cpu().numpy())


@pytest.mark.parametrize("op,dist", [("attn", "cos"), ("block", "l1")])
def test_encoder_variant_equals_chained_blocks(op, dist):
    """An encoder run scored with a variant equals rs_block_forward chained with the same
    variant (bit-exact), and its kept sets follow the oracle's variant scores."""
    import torch
    import vit_token_pruning_amd as rs
    wl = dataclasses.replace(W["deit_s"], B=6, L=97, depth=4, prune_layers=(1, 2),
                             keep_ratios=(0.7, 0.7))
    spec = spec_of(wl, op, dist)
    blocks = synth.make_encoder_weights(wl, 0)
    wd = [weights_to_dev(w, wl.dtype) for w in blocks]
    x = synth.make_input(wl, 0)
    xd = to_dev(x, wl.dtype)
    out, out_idx = rs.encoder_forward(spec, wd, xd, wl.prune_layers, wl.keep_ratios)
    torch.cuda.synchronize()
    _, ks, _ = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)
    cur, ids = xd, np.tile(np.arange(wl.L), (wl.B, 1))
    exact = total = 0
    for b in range(wl.depth):
        L = cur.shape[1]
        k = ks.get(b, L)
        cur_host = to_host(cur)
        r = rs.block_forward(spec, wd[b], cur, k)
        torch.cuda.synchronize()
        if b in ks:
            kept = r["kept_idx"].cpu().numpy()
            ora = oracle_block(cur_host, blocks[b], wl.heads, wl.ln_eps, op=op, dist=dist)
            check_scores(r["scores"].cpu().numpy(), ora["score"])
            for j in range(wl.B):
                exact += kept_admissible(kept[j], ora["score"][j], k, wl.has_cls)
                total += 1
            ids = np.take_along_axis(ids, kept.astype(np.int64), axis=1)
        cur = r["y_kept"]
    assert torch.equal(out, cur)
    assert np.array_equal(out_idx.cpu().numpy(), ids)
    print(f"encoder {op}/{dist}: exact kept-set agreement {exact}/{total}")

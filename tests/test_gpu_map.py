"""GPU parity of the attention-map baselines the pages compare against ("Representation
Shift", Sec. 3.1, Eq. (2) class-token row and Eq. (3) mean over queries, averaged over
heads): the map-forming attention kernel (its output, the stored map, both scores)
against the fp64 oracle on the same bf16/fp32 inputs; blocks and encoders scored from the
map; and the fused kernel's output through the same standalone entry point."""
import dataclasses

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, oracle_block,
                         spec_of, to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _wl(name):
    base, _, dt = name.partition("@")
    return dataclasses.replace(W[base], dtype=dt) if dt else W[base]


def _qkv(wl, B, L, seed):
    """Seeded Q|K|V rows [B, L, 3C] with peaky softmaxes (logit std ~2), rounded to the
    workload's storage type so that the oracle sees the GPU's inputs."""
    rng = np.random.default_rng([seed, 77])
    a = (rng.standard_normal((B, L, 3 * wl.C)) * 1.4).astype(np.float32)
    return synth.round_to_bf16(a) if wl.dtype == "bf16" else a


def _oracle_heads(qkv_b, heads):
    """Per head: the map A [L, L] and the output A v [L, 64] of one sample."""
    L, C3 = qkv_b.shape
    C = C3 // 3
    maps, outs = [], []
    for h in range(heads):
        q = qkv_b[:, h * 64:(h + 1) * 64].astype(np.float64)
        k = qkv_b[:, C + h * 64:C + (h + 1) * 64].astype(np.float64)
        v = qkv_b[:, 2 * C + h * 64:2 * C + (h + 1) * 64].astype(np.float64)
        a = O.softmax_rows(q @ k.T / 8.0)
        maps.append(a)
        outs.append(O.attention_materialised(q, k, v))
    return np.stack(maps), np.concatenate(outs, axis=1)


CASES = [("deit_t_block", 2, 197), ("deit_s", 3, 197), ("deit_s", 2, 138), ("deit_s@f32", 2, 65),
         ("umt_b", 1, 1568), ("deit_s", 2, 1), ("deit_s", 2, 64), ("umt_l@f32", 1, 98),
         # grids of >= 512 two-group workgroups: the fused kernel runs 32 queries per wave
         ("deit_s", 96, 197), ("deit_s@f32", 96, 130), ("umt_b", 12, 1568)]


@pytest.mark.parametrize("name,B,L", CASES)
def test_attention_map_kernel_matches_oracle(name, B, L):
    import torch
    import vit_token_pruning_amd as rs
    wl = _wl(name)
    spec = spec_of(wl)
    qkv = _qkv(wl, B, L, L)
    qd = to_dev(qkv, wl.dtype)
    out_f, _, _, _ = rs.attention(spec, qd)                                  # fused
    out_m, amap, sc, sm = rs.attention(spec, qd, want_map=True, want_cls=True, want_mean=True)
    torch.cuda.synchronize()
    out_f, out_m, amap = to_host(out_f), to_host(out_m), to_host(amap)
    sc, sm = sc.cpu().numpy(), sm.cpu().numpy()
    lpad = (L + 7) // 8 * 8
    assert amap.shape == (B, wl.heads, L, lpad)
    for b in sorted({0, B - 1}):
        maps, o = _oracle_heads(qkv[b], wl.heads)
        tol_o = (2.0 ** -7 if wl.dtype == "bf16" else 1e-5) * np.abs(o).max()
        for got in (out_f[b], out_m[b]):
            assert np.abs(got - o).max() <= tol_o, np.abs(got - o).max()
        # the stored map: one rounding of each probability, padding keys zero
        err = np.abs(amap[b][:, :, :L] - maps)
        bound = (2.0 ** -8 if wl.dtype == "bf16" else 1e-5) * maps + 1e-7
        assert (err <= bound).all(), err.max()
        assert not amap[b][:, :, L:].any()
        # Eq. (2) / Eq. (3) averaged over heads
        rel = 1e-3 if wl.dtype == "bf16" else 1e-5
        np.testing.assert_allclose(sc[b], O.attention_map_score(maps, "cls"), rtol=rel)
        np.testing.assert_allclose(sm[b], O.attention_map_score(maps, "mean"), rtol=rel)
        assert abs(sm[b].sum() - 1.0) < 1e-4


SHAPES = [("deit_t_block", 2, 197, 0.7), ("deit_s", 3, 138, 0.7), ("deit_s@f32", 2, 97, 0.7),
          ("umt_b", 1, 392, 0.5), ("umt_l@f32", 1, 98, 0.5)]


@pytest.mark.parametrize("name,B,L,ratio", SHAPES)
@pytest.mark.parametrize("op", ["map_cls", "map_mean"])
@pytest.mark.parametrize("attn_map", [False, True])
def test_block_scored_from_map(name, B, L, ratio, op, attn_map):
    import torch
    import vit_token_pruning_amd as rs
    wl = _wl(name)
    if op == "map_cls" and not wl.has_cls:
        pytest.skip("Eq. (2) needs a class token")
    k = O.keep_count(ratio, L)
    x = synth.make_input(wl, 31 + L, B=B, L=L)
    w = synth.make_block_weights(wl, 0, 31 + L, init="full")
    spec = spec_of(wl, op, attn_map=attn_map)
    r = rs.block_forward(spec, weights_to_dev(w, wl.dtype), to_dev(x, wl.dtype), k)
    torch.cuda.synchronize()
    y, s = to_host(r["y"]), r["scores"].cpu().numpy()
    kept = r["kept_idx"].cpu().numpy()
    ora = oracle_block(x, w, wl.heads, wl.ln_eps, op=op)
    check_block_output(y, ora["x_hat"], x, wl.dtype)
    err = check_scores(s, ora["score"])
    exact = 0
    for b in range(B):
        exact += kept_admissible(kept[b], ora["score"][b], k, wl.has_cls)
        assert kept[b].tolist() == O.select_kept(s[b], k, wl.has_cls)
    if attn_map:
        # storing the map changes nothing else
        r0 = rs.block_forward(spec_of(wl, op), weights_to_dev(w, wl.dtype), to_dev(x, wl.dtype), k)
        assert np.array_equal(to_host(r0["y"]), y) and np.array_equal(r0["scores"].cpu().numpy(), s)
    print(f"{name} B{B} L{L} {op} map={attn_map}: score rel err {err:.2e}, exact kept {exact}/{B}")


@pytest.mark.parametrize("name,op,attn_map", [("deit_s", "map_cls", True), ("umt_b", "map_mean", True),
                                              ("deit_s", "map_mean", False)])
def test_encoder_scored_from_map_equals_chained_blocks(name, op, attn_map):
    """The encoder equals rs_block_forward chained over its schedule.  Without stored maps
    only the pruning blocks form their map; the chain runs the other blocks with the
    method's score, whose block calls use the fused attention the encoder uses there."""
    import torch
    import vit_token_pruning_amd as rs
    if name == "deit_s":
        wl = dataclasses.replace(W[name], B=6, L=97, depth=4, prune_layers=(1, 2), keep_ratios=(0.7, 0.7))
    else:
        wl = dataclasses.replace(W[name], B=2, L=392, depth=3, prune_layers=(0, 2), keep_ratios=(0.5, 0.5))
    spec = spec_of(wl, op, attn_map=attn_map)
    blocks = synth.make_encoder_weights(wl, 0)
    wd = [weights_to_dev(w, wl.dtype) for w in blocks]
    xd = to_dev(synth.make_input(wl, 0), wl.dtype)
    out, out_idx = rs.encoder_forward(spec, wd, xd, wl.prune_layers, wl.keep_ratios)
    torch.cuda.synchronize()
    _, ks, _ = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)
    cur, ids = xd, np.tile(np.arange(wl.L), (wl.B, 1))
    exact = total = 0
    for b in range(wl.depth):
        L = cur.shape[1]
        k = ks.get(b, L)
        cur_host = to_host(cur)
        sb = spec if (attn_map or b in ks) else spec_of(wl)
        r = rs.block_forward(sb, wd[b], cur, k)
        torch.cuda.synchronize()
        if b in ks:
            kept = r["kept_idx"].cpu().numpy()
            ora = oracle_block(cur_host, blocks[b], wl.heads, wl.ln_eps, op=op)
            check_scores(r["scores"].cpu().numpy(), ora["score"])
            for j in range(wl.B):
                exact += kept_admissible(kept[j], ora["score"][j], k, wl.has_cls)
                total += 1
            ids = np.take_along_axis(ids, kept.astype(np.int64), axis=1)
        cur = r["y_kept"]
    assert torch.equal(out, cur)
    assert np.array_equal(out_idx.cpu().numpy(), ids)
    print(f"encoder {name} {op} map={attn_map}: exact kept-set agreement {exact}/{total}")

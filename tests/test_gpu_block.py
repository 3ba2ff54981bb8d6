"""GPU parity of one pre-LN block with scoring and selection (rs_block_forward)
against the fp64 oracle, at every stage shape of the workloads (small batch, several
tiles and a ragged tail), with the closed forms and the self-consistency invariants."""
import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, oracle_block,
                         spec_of, to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
# (workload, batch, stage length, keep ratio)
CASES = [("deit_t_block", 2, 197, 0.7)]
CASES += [("deit_s", 3, L, 0.7) for L in (197, 138, 97, 68)]
CASES += [("deit_b", 2, L, 0.65) for L in (197, 128, 83, 54)]
CASES += [("umt_b", 1, L, 0.5) for L in (1568, 784, 392, 196)]
CASES += [("umt_l", 1, L, 0.5) for L in (1568, 784, 392, 196, 98)]
# fp32 with K split (fc2 at DeiT-S widths; all four GEMMs at UMT-L widths)
CASES += [("deit_s@f32", 2, 97, 0.7), ("umt_l@f32", 1, 98, 0.5)]


def _wl(name):
    """A workload by name; `name@f32` is the same architecture computed in fp32."""
    import dataclasses
    base, _, dt = name.partition("@")
    return dataclasses.replace(W[base], dtype=dt) if dt else W[base]


def _block(wl, B, L, k, init, seed, zero=(), spread=False):
    import torch
    import vit_token_pruning_amd as rs
    x = synth.make_input(wl, seed, B=B, L=L, spread=spread)
    w = synth.make_block_weights(wl, 0, seed, init=init, zero=zero)
    spec = spec_of(wl)
    wd = weights_to_dev(w, wl.dtype)
    r = rs.block_forward(spec, wd, to_dev(x, wl.dtype), k)
    torch.cuda.synchronize()
    return x, w, {key: (None if v is None else v) for key, v in r.items()}


@pytest.mark.parametrize("name,B,L,ratio", CASES)
@pytest.mark.parametrize("init", ["full", "paper"])
def test_block_matches_oracle(name, B, L, ratio, init):
    import vit_token_pruning_amd as rs
    wl = _wl(name)
    k = O.keep_count(ratio, L)
    seed = 11 + L
    x, w, r = _block(wl, B, L, k, init, seed)
    y, s = to_host(r["y"]), r["scores"].cpu().numpy()
    kept, yk = r["kept_idx"].cpu().numpy(), to_host(r["y_kept"])
    ora = oracle_block(x, w, wl.heads, wl.ln_eps)
    check_block_output(y, ora["x_hat"], x, wl.dtype)
    check_scores(s, ora["score"])
    exact = 0
    for b in range(B):
        exact += kept_admissible(kept[b], ora["score"][b], k, wl.has_cls)
        # self-consistency: exact top-k of the GPU's own scores, rows gathered bit-exactly
        assert kept[b].tolist() == O.select_kept(s[b], k, wl.has_cls)
        np.testing.assert_array_equal(yk[b], y[b][kept[b]])
    print(f"{name} B{B} L{L} k{k} {init}: exact kept-set agreement {exact}/{B}")
    # determinism: a second call is bit-identical
    r2 = rs.block_forward(spec_of(wl), weights_to_dev(w, wl.dtype), to_dev(x, wl.dtype), k)
    assert np.array_equal(to_host(r2["y"]), y) and np.array_equal(r2["scores"].cpu().numpy(), s)
    assert np.array_equal(r2["kept_idx"].cpu().numpy(), kept)


@pytest.mark.parametrize("name,L", [("deit_t_block", 197), ("deit_s", 138), ("umt_l", 392)])
def test_zero_branches_closed_forms(name, L):
    wl = W[name]
    B, k = 2, O.keep_count(0.5, L)
    # attention and MLP branches zero: x_hat = x exactly, score = ||x||
    x, w, r = _block(wl, B, L, k, "full", 3, zero=("w_proj", "b_proj", "w_fc2", "b_fc2"))
    np.testing.assert_array_equal(to_host(r["y"]), x)
    want = np.linalg.norm(x.astype(np.float64), axis=-1)
    s = r["scores"].cpu().numpy()
    assert (np.abs(s - want) / want).max() <= 1e-4
    for b in range(B):
        assert r["kept_idx"][b].cpu().tolist() == O.select_kept(s[b], k, wl.has_cls)
    # MLP branch zero: x_hat = x', score = ||x'||
    x, w, r = _block(wl, B, L, k, "full", 4, zero=("w_fc2", "b_fc2"))
    ora = oracle_block(x, w, wl.heads, wl.ln_eps)
    np.testing.assert_allclose(ora["score"], np.linalg.norm(ora["x_prime"], axis=-1), rtol=1e-12)
    check_block_output(to_host(r["y"]), ora["x_prime"], x, wl.dtype)
    check_scores(r["scores"].cpu().numpy(), ora["score"])


def test_keep_all_is_identity_and_spread_inputs():
    wl = W["deit_s"]
    x, w, r = _block(wl, 2, 97, 97, "full", 5)
    assert r["kept_idx"].cpu().numpy().tolist() == [list(range(97))] * 2
    assert np.array_equal(to_host(r["y_kept"]), to_host(r["y"]))
    # spread rows (a_i ~ U(0.5, 1.5)) shrink the tie band: report exact agreement
    k = O.keep_count(0.7, 197)
    x, w, r = _block(wl, 4, 197, k, "paper", 6, spread=True)
    ora = oracle_block(x, w, wl.heads, wl.ln_eps)
    check_scores(r["scores"].cpu().numpy(), ora["score"])
    kept = r["kept_idx"].cpu().numpy()
    exact = sum(kept_admissible(kept[b], ora["score"][b], k, True) for b in range(4))
    print(f"spread inputs: exact kept-set agreement {exact}/4")

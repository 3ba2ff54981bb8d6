"""GPU edge cases of one block with scoring and selection against the fp64 oracle: the
smallest inputs (one token, one sample, keep one token) and the longest sequence the ABI
accepts (RS_MAX_TOKENS tokens in one sample: attention over 16384 keys, the 1024-thread
top-k)."""
import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, oracle_block,
                         spec_of, to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu


def _run(wl, B, L, k, seed):
    import torch
    import vit_token_pruning_amd as rs
    x = synth.make_input(wl, seed, B=B, L=L)
    w = synth.make_block_weights(wl, 0, seed, init="full")
    r = rs.block_forward(spec_of(wl), weights_to_dev(w, wl.dtype), to_dev(x, wl.dtype), k)
    torch.cuda.synchronize()
    return x, w, r


@pytest.mark.parametrize("name", ["deit_s", "deit_t_block"])
@pytest.mark.parametrize("B,L,k", [(1, 1, 1), (1, 2, 1), (3, 1, 1), (2, 3, 2), (1, 65, 33), (5, 2, 2)])
def test_tiny_blocks(name, B, L, k):
    """One-token rows attend only to themselves; with a class token and k = 1 only the
    class token survives; K splits at M = 1."""
    wl = synth.WORKLOADS[name]
    x, w, r = _run(wl, B, L, k, 40 + L)
    y, s, kept = to_host(r["y"]), r["scores"].cpu().numpy(), r["kept_idx"].cpu().numpy()
    ora = oracle_block(x, w, wl.heads, wl.ln_eps)
    check_block_output(y, ora["x_hat"], x, wl.dtype)
    check_scores(s, ora["score"])
    for b in range(B):
        kept_admissible(kept[b], ora["score"][b], k, wl.has_cls)
        assert kept[b].tolist() == O.select_kept(s[b], k, wl.has_cls)
        np.testing.assert_array_equal(to_host(r["y_kept"])[b], y[b][kept[b]])
    if k == 1 and wl.has_cls:
        assert (kept == 0).all()


def test_longest_sequence():
    """RS_MAX_TOKENS tokens (16384) in one sample at C = 64 (one head), bf16: the whole
    block and the kept set against the oracle."""
    import vit_token_pruning_amd as rs  # noqa: F401  (the library must load)
    wl = synth.Workload("long", 1, 16384, 64, 1, 256, 1, "bf16", False, (0,), (0.5,), "x")
    k = O.keep_count(0.5, wl.L)
    x, w, r = _run(wl, 1, wl.L, k, 3)
    ora = O.block_forward(x[0], w, wl.heads, wl.ln_eps)
    check_block_output(to_host(r["y"])[0], ora["x_hat"], x[0], wl.dtype)
    s = r["scores"].cpu().numpy()[0]
    check_scores(s, ora["score"])
    kept = r["kept_idx"].cpu().numpy()[0]
    exact = kept_admissible(kept, ora["score"], k, False)
    assert kept.tolist() == O.select_kept(s, k, False)
    print(f"L = 16384: exact kept-set agreement {exact}")

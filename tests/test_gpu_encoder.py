"""Full-size encoder parity (the four encoder workloads at their real batch and length,
the launch configuration the benchmark times).

rs_encoder_forward is checked bit-exactly against a chain of rs_block_forward calls at
the same shapes (same kernels, deterministic), whose per-block results are checked
against the oracle on sampled samples with teacher forcing: the oracle block is fed the
GPU's own block input, so each comparison measures one block's rounding."""
import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, spec_of, to_dev,
                         to_host, weights_to_dev)

pytestmark = pytest.mark.gpu

SAMPLED = {"deit_s": [0, 255], "deit_b": [0, 127], "umt_b": [5], "umt_l": [2]}


@pytest.mark.parametrize("name", ["deit_s", "deit_b", "umt_b", "umt_l"])
def test_encoder_full_size(name):
    import torch
    import vit_token_pruning_amd as rs
    wl = synth.WORKLOADS[name]
    spec = spec_of(wl)
    x = synth.make_input(wl, 0)
    blocks = synth.make_encoder_weights(wl, 0)
    wd = [weights_to_dev(w, wl.dtype) for w in blocks]
    xd = to_dev(x, wl.dtype)
    lens, ks, L_final = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)

    out, out_idx = rs.encoder_forward(spec, wd, xd, wl.prune_layers, wl.keep_ratios)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (wl.B, L_final, wl.C)

    samp = SAMPLED[name]
    cur = xd
    ids = np.tile(np.arange(wl.L), (wl.B, 1))
    exact = total = 0
    for b in range(wl.depth):
        L = cur.shape[1]
        k = ks.get(b, L)
        cur_host = to_host(cur[samp])
        r = rs.block_forward(spec, wd[b], cur, k)
        torch.cuda.synchronize()
        y = to_host(r["y"][samp])
        s = r["scores"][samp].cpu().numpy()
        kept_all = r["kept_idx"].cpu().numpy()
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
    assert torch.equal(out, cur), "encoder output differs from the chained blocks"
    assert np.array_equal(out_idx.cpu().numpy(), ids)
    print(f"{name}: exact kept-set agreement {exact}/{total} sampled prune stages")

"""GPU parity of one block over a seeded grid of shapes the named workloads do not cover:
widths 64 .. 1024 (one to sixteen heads, 128-column tiles with a ragged last tile when
C is not a multiple of 128), MLP ratios 2 and 4, token counts from 2 to 300 (ragged row
tiles, ragged key tiles, query blocks with idle waves), batches of 1 to 5, with and
without a class token, in bf16 and fp32."""
import dataclasses

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import (check_block_output, check_scores, kept_admissible, oracle_block,
                         spec_of, to_dev, to_host, weights_to_dev)

pytestmark = pytest.mark.gpu


def _cases(n=24):
    rng = np.random.default_rng(2024)
    out = []
    for i in range(n):
        C = int(rng.choice([64, 128, 192, 256, 320, 448, 512, 768, 1024]))
        ratio = int(rng.choice([2, 4]))
        L = int(rng.integers(2, 301))
        B = int(rng.integers(1, 6))
        dt = "f32" if i % 3 == 0 else "bf16"
        cls = bool(i % 2)
        keep = float(rng.choice([0.5, 0.7, 0.9]))
        out.append((i, C, ratio, L, B, dt, cls, keep))
    return out


@pytest.mark.parametrize("i,C,ratio,L,B,dt,cls,keep", _cases())
def test_block_shape_grid(i, C, ratio, L, B, dt, cls, keep):
    import torch
    import vit_token_pruning_amd as rs
    wl = synth.Workload(f"grid{i}", B, L, C, C // 64, ratio * C, 1, dt, cls, (0,), (keep,), "x")
    k = max(1, O.keep_count(keep, L))
    x = synth.make_input(wl, 100 + i, spread=True)
    w = synth.make_block_weights(wl, 0, 100 + i, init="full")
    r = rs.block_forward(spec_of(wl), weights_to_dev(w, dt), to_dev(x, dt), k)
    torch.cuda.synchronize()
    y, s = to_host(r["y"]), r["scores"].cpu().numpy()
    kept, yk = r["kept_idx"].cpu().numpy(), to_host(r["y_kept"])
    ora = oracle_block(x, w, wl.heads, wl.ln_eps)
    check_block_output(y, ora["x_hat"], x, dt)
    check_scores(s, ora["score"])
    for b in range(B):
        kept_admissible(kept[b], ora["score"][b], k, cls)
        assert kept[b].tolist() == O.select_kept(s[b], k, cls)
        np.testing.assert_array_equal(yk[b], y[b][kept[b]])

"""Helpers shared by the GPU parity tests: moving seeded inputs to the device, running
the oracle per sample, and the agreement rules (tolerances written here)."""
from __future__ import annotations

import numpy as np

from oracle import rs_oracle as O

# Agreement rules (per block):
SCORE_REL = 1e-2          # |s_gpu - s_ora| <= 1e-2 * s_ora for every token
BAND_REL = 1e-2           # tie band around the k-th score for the kept-set rule
BF16_OUT_ABS = 2e-2       # max |x_hat_gpu - x_hat_ora| <= 2e-2 * RMS(block input), bf16,
                          # plus half a bf16 ulp of the stored value (its own rounding)
F32_OUT_REL = 1e-4        # max |x_hat_gpu - x_hat_ora| <= 1e-4 * max |x_hat_ora|, fp32


def torch_dtype(dt):
    import torch
    return torch.bfloat16 if dt == "bf16" else torch.float32


def to_dev(a: np.ndarray, dt: str):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(torch_dtype(dt))


def weights_to_dev(w, dt):
    return {k: to_dev(v, dt) for k, v in w.items()}


def to_host(t) -> np.ndarray:
    return t.float().cpu().numpy()


def spec_of(wl, op: str = "mlp", dist: str = "l2", attn_map: bool = False):
    import vit_token_pruning_amd as rs
    return rs.ModelSpec(wl.C, wl.heads, wl.hidden, torch_dtype(wl.dtype), wl.has_cls, wl.ln_eps,
                        score_op=op, score_dist=dist, attn_map=attn_map)


def oracle_block(x: np.ndarray, w, heads: int, eps: float, samples=None, op: str = "mlp",
                 dist: str = "l2"):
    """Oracle block per sample of x [B, L, C] (float64 results stacked)."""
    samples = range(x.shape[0]) if samples is None else samples
    res = [O.block_forward(x[b], w, heads, eps, op=op, dist=dist) for b in samples]
    return {k: np.stack([r[k] for r in res]) for k in ("x_prime", "mlp", "x_hat", "score")}


def check_scores(s_gpu: np.ndarray, s_ora: np.ndarray):
    err = np.abs(s_gpu.astype(np.float64) - s_ora) / np.maximum(s_ora, 1e-30)
    assert err.max() <= SCORE_REL, f"score rel err {err.max():.3e}"
    return float(err.max())


def kept_admissible(kept_gpu: np.ndarray, s_ora: np.ndarray, k: int, has_cls: bool):
    """Kept-set rule for one sample: exact outside the band of tokens whose oracle score
    lies within BAND_REL of the k-th largest unforced score.  Returns True if the sets
    agree exactly."""
    kept_gpu = [int(i) for i in kept_gpu]
    assert len(kept_gpu) == k
    assert kept_gpu == sorted(set(kept_gpu)), "kept indices not unique ascending"
    L = len(s_ora)
    assert all(0 <= i < L for i in kept_gpu)
    if has_cls:
        assert kept_gpu[0] == 0, "class token dropped"
    ora = O.select_kept(s_ora, k, has_cls)
    unforced = s_ora[1:] if has_cls else s_ora
    kk = k - (1 if has_cls else 0)
    if kk == 0 or kk == len(unforced):
        assert kept_gpu == ora
        return True
    sk = np.sort(unforced)[::-1][kk - 1]
    band = {i for i in range(L) if not (has_cls and i == 0) and abs(s_ora[i] - sk) <= BAND_REL * sk}
    assert set(kept_gpu) - band == set(ora) - band, "kept set differs outside the tie band"
    return kept_gpu == ora


def bf16_half_ulp(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bf16 values (8 significant bits) in the binade of |v|: the most
    that rounding a real number to the nearest bf16 value v can move it."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def check_block_output(y_gpu: np.ndarray, y_ora: np.ndarray, x_in: np.ndarray, dt: str):
    """bf16: the block's arithmetic error is bounded by 2e-2 * RMS(block input), and the
    stored output is that result rounded to bf16, so each element may lie a further half
    bf16 ulp (of its own magnitude) from the oracle's exact value -- for |x_hat| >= 8 at
    RMS(x) ~ 1.5 that storage rounding alone (up to 2^-5) exceeds the arithmetic bound.
    fp32: 1e-4 * max |x_hat_ora| (norm-wise relative)."""
    y = np.asarray(y_gpu, np.float64)
    err = np.abs(y - y_ora)
    if dt == "bf16":
        tol = BF16_OUT_ABS * float(np.sqrt(np.mean(np.asarray(x_in, np.float64) ** 2)))
        d = float((err - bf16_half_ulp(y)).max())
        assert d <= tol, (f"block output err beyond the stored value's half ulp {d:.3e} > {tol:.3e} "
                          f"(max raw err {err.max():.3e})")
    else:
        tol = F32_OUT_REL * float(np.abs(y_ora).max())
        d = float(err.max())
        assert d <= tol, f"block output max err {d:.3e} > {tol:.3e}"
    return d, tol

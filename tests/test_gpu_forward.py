"""GPU parity of the steps around the encoder (the tokenisation of "Representation Shift",
Sec. 3.1, and the final LayerNorm + head of the DeiT / UMT models the pages run): the
patch embedding and the head against the fp64 oracle, and the whole forward pass
(rs_vit_forward) against the chain patch_embed -> encoder_forward -> head bit for bit,
with the chain's stages checked against the oracle (teacher forcing)."""
import dataclasses

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import check_block_output, spec_of, to_dev, to_host, weights_to_dev

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def _wl(name):
    base, _, dt = name.partition("@")
    return dataclasses.replace(W[base], dtype=dt) if dt else W[base]


def _img(g):
    import vit_token_pruning_amd as rs
    return rs.ImageSpec(g.frames, g.in_chans, g.height, g.width, g.patch)


def check_rows(got, want, dt):
    """Rows stored once in bf16 after fp32 arithmetic: within one rounding (2^-9
    relative, with margin 2^-8) plus fp32 accumulation; fp32: 1e-5 of the largest."""
    got, want = got.astype(np.float64), np.asarray(want, np.float64)
    err = np.abs(got - want)
    if dt == "bf16":
        bound = 2.0 ** -8 * np.abs(want) + 1e-4 * float(np.sqrt(np.mean(want ** 2)))
        assert (err <= bound).all(), f"max err {err.max():.3e}"
    else:
        assert err.max() <= 1e-5 * np.abs(want).max(), f"max err {err.max():.3e}"


def check_logits(got, want, dt):
    got, want = got.astype(np.float64), np.asarray(want, np.float64)
    d = np.abs(got - want).max()
    tol = (2e-2 * float(np.sqrt(np.mean(want ** 2))) if dt == "bf16"
           else 1e-4 * float(np.abs(want).max()))
    assert d <= tol, f"logits max err {d:.3e} > {tol:.3e}"


# (workload, geometry overrides, batch): DeiT-T fp32 (split over K), DeiT-S bf16 (one
# tile column per 128 channels, ragged M), a 2-frame clip without class token, patch 8
# and 32 on non-square images, and a batch large enough for the direct path
PATCH_CASES = [
    ("deit_t_block", {}, 2),
    ("deit_s", {}, 3),
    ("umt_b", {"frames": 2}, 2),
    ("deit_s", {"height": 64, "width": 96, "patch": 8}, 3),
    ("deit_s@f32", {"height": 64, "width": 96, "patch": 8}, 2),
    ("umt_l", {"frames": 1, "height": 96, "width": 64, "patch": 32}, 3),
    ("deit_s", {}, 64),
]


@pytest.mark.parametrize("name,over,B", PATCH_CASES)
def test_patch_embed_matches_oracle(name, over, B):
    import torch
    import vit_token_pruning_amd as rs
    wl = _wl(name)
    g = dataclasses.replace(synth.Geometry(1, 3, 224, 224, 16, 8, "cls"), **over)
    images = synth.make_images(wl, g, 4, B=B)
    emb = synth.make_embed_weights(wl, g, 4)
    tok = rs.patch_embed(spec_of(wl), _img(g), weights_to_dev(emb, wl.dtype), to_dev(images, wl.dtype))
    torch.cuda.synchronize()
    got = to_host(tok)
    assert got.shape == (B, g.tokens(wl.has_cls), wl.C)
    for b in sorted({0, B - 1}):
        want = O.patch_embed(images[b], emb["w_patch"], emb["b_patch"],
                             emb["cls"] if wl.has_cls else None, emb["pos"], g.patch)
        check_rows(got[b], want, wl.dtype)


@pytest.mark.parametrize("name,L,pool,n_out,B", [
    ("deit_s", 68, "cls", 1000, 5), ("deit_t_block", 138, "cls", 1000, 3),
    ("umt_l", 98, "mean", 512, 4), ("umt_b@f32", 392, "mean", 512, 2), ("deit_s", 197, "mean", 8, 3),
    ("umt_l", 1205, "mean", 512, 2),
])
@pytest.mark.parametrize("init", ["paper", "full"])
def test_head_matches_oracle(name, L, pool, n_out, B, init):
    import torch
    import vit_token_pruning_amd as rs
    wl = _wl(name)
    g = synth.Geometry(1, 3, 224, 224, 16, n_out, pool)
    x = synth.make_input(wl, 9, B=B, L=L, spread=True)
    hw = synth.make_head_weights(wl, g, 9, init)
    feat, logits = rs.head(spec_of(wl), weights_to_dev(hw, wl.dtype), to_dev(x, wl.dtype), pool)
    torch.cuda.synchronize()
    f, lg = to_host(feat), to_host(logits)
    for b in range(B):
        wf, wlg = O.head(x[b], hw["ln_g"], hw["ln_b"], hw["w_head"], hw["b_head"], pool, wl.ln_eps)
        check_rows(f[b], wf, wl.dtype)
        check_logits(lg[b], wlg, wl.dtype)


def _forward_and_chain(wl, g, B, samples, seed=0):
    """rs_vit_forward, and the chain of its stages, with the stages checked against the
    oracle on `samples` (each fed the GPU's own input)."""
    import torch
    import vit_token_pruning_amd as rs
    spec, img = spec_of(wl), _img(g)
    images = synth.make_images(wl, g, seed, B=B)
    emb = synth.make_embed_weights(wl, g, seed)
    blocks = synth.make_encoder_weights(wl, seed)
    hw = synth.make_head_weights(wl, g, seed)
    ed, wd, hd = weights_to_dev(emb, wl.dtype), [weights_to_dev(w, wl.dtype) for w in blocks], \
        weights_to_dev(hw, wl.dtype)
    imd = to_dev(images, wl.dtype)
    feat, logits, idx = rs.vit_forward(spec, img, ed, wd, hd, g.pool, imd, wl.prune_layers,
                                       wl.keep_ratios)
    torch.cuda.synchronize()
    tok = rs.patch_embed(spec, img, ed, imd)
    enc, enc_idx = rs.encoder_forward(spec, wd, tok, wl.prune_layers, wl.keep_ratios)
    f2, lg2 = rs.head(spec, hd, enc, g.pool)
    torch.cuda.synchronize()
    assert torch.equal(feat, f2) and torch.equal(logits, lg2), "forward differs from its chain"
    assert torch.equal(idx, enc_idx)
    tok_h, enc_h, f_h, lg_h = to_host(tok), to_host(enc), to_host(f2), to_host(lg2)
    for b in samples:
        want = O.patch_embed(images[b], emb["w_patch"], emb["b_patch"],
                             emb["cls"] if wl.has_cls else None, emb["pos"], g.patch)
        check_rows(tok_h[b], want, wl.dtype)
        wf, wlg = O.head(enc_h[b], hw["ln_g"], hw["ln_b"], hw["w_head"], hw["b_head"], g.pool,
                         wl.ln_eps)
        check_rows(f_h[b], wf, wl.dtype)
        check_logits(lg_h[b], wlg, wl.dtype)
    return images, emb, blocks, hw, idx.cpu().numpy(), lg_h


@pytest.mark.parametrize("name,B,depth", [("deit_s", 4, 4), ("deit_t_block", 2, 1), ("umt_b", 2, 3)])
def test_vit_forward_small(name, B, depth):
    """Small batches (one lane), with the whole pass also run by the oracle end to end on
    one sample for the fp32 case."""
    wl = W[name]
    if name == "umt_b":
        wl = dataclasses.replace(wl, L=392, depth=depth, prune_layers=(0, 1), keep_ratios=(0.5, 0.5))
        g = synth.Geometry(2, 3, 224, 224, 16, 512, "mean")
    else:
        wl = dataclasses.replace(wl, depth=depth, prune_layers=tuple(p for p in (0, 2) if p < depth),
                                 keep_ratios=(0.7, 0.8)[:len([p for p in (0, 2) if p < depth])])
        g = synth.geometry(wl)
    images, emb, blocks, hw, idx, logits = _forward_and_chain(wl, g, B, [0, B - 1])
    if wl.dtype == "f32":
        # end to end in fp64 without teacher forcing: at fp32 the selections agree and
        # the logits match to the fp32 rule
        feat, lg, ids = O.vit_forward(images[0], emb, blocks, hw, wl.heads, g.patch,
                                      wl.prune_layers, wl.keep_ratios, wl.has_cls, g.pool,
                                      wl.ln_eps)
        assert ids.tolist() == idx[0].tolist()
        check_logits(logits[0], lg, wl.dtype)


@pytest.mark.parametrize("name", ["deit_s", "umt_b"])
def test_vit_forward_full_size(name):
    """The benchmark's whole-forward configuration (two encoder lanes at DeiT-S batch 256;
    UMT-B 8 clips of 8 frames), bit-exact against the chain, sampled stages against the
    oracle."""
    wl = W[name]
    _forward_and_chain(wl, synth.geometry(wl), wl.B, [wl.B - 1])

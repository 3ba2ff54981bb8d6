"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Each test checks the oracle against something the pages or mathematics fix: the
GFLOPs the pages print, textbook values, closed forms, identities and brute force
on tiny inputs.  They are chosen so that a plausible slip (dropped term, wrong sign,
wrong scale, transposed operand, wrong tie order, wrong schedule reading) fails one.
Page cited throughout: "Representation Shift: Unifying Token Compression with
FlashAttention" (arXiv HTML).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- work model / schedule

def _tol(printed):
    # printed to one decimal (+-0.05) plus 0.2% for terms the pages count and the
    # model leaves out (final norm, head)
    return 0.05 + 0.002 * printed


def test_flop_model_reproduces_printed_gflops():
    """Tables 2, 4, 5 GFLOPs: reproduced only by compounding post-block pruning."""
    for e in _gold("gflops_printed.json")["entries"]:
        g = O.encoder_gmacs(e["depth"], e["L"], e["C"], e["prune"], e["keep"], e["patches"])
        assert abs(g - e["printed"]) <= _tol(e["printed"]), (e["cite"], g)


def test_flop_model_rejects_other_schedule_readings():
    """0-based [1,4,7] and fixed-count pruning miss Table 5 for DeiT-S and DeiT-B."""
    ents = [e for e in _gold("gflops_printed.json")["entries"]
            if e["model"] in ("DeiT-S", "DeiT-B") and e["prune"]]
    assert len(ents) == 2
    for e in ents:
        g0 = O.encoder_gmacs(e["depth"], e["L"], e["C"], [1, 4, 7], e["keep"], e["patches"])
        assert abs(g0 - e["printed"]) > _tol(e["printed"])
        # fixed count: drop 20% of the *original* tokens at each prune block
        r = round(0.2 * e["L"])
        lens = [e["L"]] + [e["L"] - r] * 3 + [e["L"] - 2 * r] * 3 + [e["L"] - 3 * r] * 5
        gf = (sum(O.block_macs(l, e["C"]) for l in lens) + e["patches"] * 768 * e["C"]) / 1e9
        assert abs(gf - e["printed"]) > _tol(e["printed"])


def test_schedules_of_the_workloads():
    assert O.schedule(1, 197, [0], [0.7])[1] == {0: 138}
    assert O.schedule(12, 197, [3, 6, 9], [0.7] * 3)[1] == {3: 138, 6: 97, 9: 68}
    assert O.schedule(12, 197, [2, 5, 8], [0.65] * 3)[1] == {2: 128, 5: 83, 8: 54}
    assert O.schedule(12, 1568, [1, 4, 7], [0.5] * 3)[1] == {1: 784, 4: 392, 7: 196}
    assert O.schedule(24, 1568, [2, 6, 10, 14], [0.5] * 4)[1] == {2: 784, 6: 392, 10: 196, 14: 98}
    # round half up, in double: 0.5 * 3 = 1.5 -> 2 ; 0.9 * 1905 = 1714.5 -> 1715
    assert O.keep_count(0.5, 3) == 2 and O.keep_count(0.9, 1905) == 1715


# ---------------------------------------------------------------- elementwise pieces

def test_gelu_is_the_erf_form():
    for p in _gold("gelu_values.json")["points"]:
        assert abs(O.gelu(np.array([p["z"]]))[0] - p["z"] * p["phi"]) < 1e-13
    g1 = O.gelu(np.array([1.0]))[0]
    tanh_form = 0.5 * (1 + math.tanh(math.sqrt(2 / math.pi) * (1 + 0.044715)))
    assert abs(g1 - tanh_form) > 1e-4
    z = np.linspace(-6, 6, 101)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(O.gelu(z) - O.gelu(-z), z, atol=1e-14)


def test_layer_norm_closed_forms():
    g = np.array([2.0, 3.0, 5.0, 7.0])
    b = np.array([0.5, -1.0, 0.25, 4.0])
    # constant row -> beta (a gamma/beta swap gives gamma)
    np.testing.assert_allclose(O.layer_norm(np.full((1, 4), 3.3), g, b, 1e-6)[0], b, atol=1e-9)
    # [1,-1,1,-1]: mean 0, biased variance 1 -> z / sqrt(1 + eps); eps = 0.5 separates
    # biased from unbiased variance and sqrt(var + eps) from sqrt(var) + eps
    z = np.array([[1.0, -1.0, 1.0, -1.0]])
    out = O.layer_norm(z, np.ones(4), np.zeros(4), 0.5)
    np.testing.assert_allclose(out, z / math.sqrt(1.5), rtol=1e-14)
    # affine applied per channel after normalisation
    np.testing.assert_allclose(O.layer_norm(z, g, b, 0.5), z / math.sqrt(1.5) * g + b, rtol=1e-14)
    # random rows: mean 0, variance sigma^2 / (sigma^2 + eps)
    r = np.random.default_rng(3).standard_normal((7, 64)) * 0.3 + 2
    eps = 1e-2
    o = O.layer_norm(r, np.ones(64), np.zeros(64), eps)
    np.testing.assert_allclose(o.mean(axis=1), 0, atol=1e-12)
    np.testing.assert_allclose(o.var(axis=1), r.var(axis=1) / (r.var(axis=1) + eps), rtol=1e-12)


def test_linear_orientation_is_out_by_in():
    z = np.random.default_rng(0).standard_normal((5, 6))
    w = np.zeros((4, 6))
    w[2, 5] = 1.0
    b = np.array([0.0, 0.0, 0.125, 0.0])
    y = O.linear(z, w, b)
    np.testing.assert_array_equal(y[:, 2], z[:, 5] + 0.125)
    assert not y[:, [0, 1, 3]].any()


# ---------------------------------------------------------------- attention (Eq. 1)

def test_fused_attention_equals_materialised():
    rng = np.random.default_rng(1)
    for L, d in [(1, 64), (7, 64), (70, 64), (197, 64), (33, 8)]:
        q, k, v = (rng.standard_normal((L, d)) * 2 for _ in range(3))
        ref = O.attention_materialised(q, k, v)
        for blk in (1, 5, 32, L):
            np.testing.assert_allclose(O.attention_online(q, k, v, blk), ref, rtol=1e-12, atol=1e-13)


def test_attention_special_cases():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((1, 64))
    np.testing.assert_allclose(O.attention_materialised(rng.standard_normal((1, 64)),
                                                        rng.standard_normal((1, 64)), v), v)
    # Q = 0: every key weighs 1/L, the output is the mean value row
    k, v = rng.standard_normal((9, 64)), rng.standard_normal((9, 64))
    np.testing.assert_allclose(O.attention_materialised(np.zeros((3, 64)), k, v),
                               np.tile(v.mean(0), (3, 1)), rtol=1e-13)
    # two keys: weight of key 0 is the logistic of (q.k0 - q.k1)/sqrt(d), d = 64
    q = np.zeros((1, 64)); q[0, 0] = 1.0
    k = np.zeros((2, 64)); k[0, 0] = 3.0; k[1, 0] = -1.0
    v = np.array([[1.0] + [0.0] * 63, [0.0] * 63 + [1.0]])
    w0 = 1.0 / (1.0 + math.exp(-(3.0 - (-1.0)) / 8.0))
    o = O.attention_materialised(q, k, v)
    assert abs(o[0, 0] - w0) < 1e-14 and abs(o[0, 63] - (1 - w0)) < 1e-14


def test_multi_head_split_is_consecutive_columns():
    # C = 8, two heads of 4.  Head 0 sees one-hot tokens with a large Q/K gain -> attends to
    # itself; head 1 has Q = K = 0 -> uniform.  V = identity.
    L, C, H = 4, 8, 2
    xn = np.zeros((L, C))
    xn[np.arange(L), np.arange(L)] = 1.0
    xn[:, 4:] = np.random.default_rng(4).standard_normal((L, 4))
    w = np.zeros((3 * C, C))
    w[0:4, 0:4] = 30.0 * np.eye(4)          # Q, head 0
    w[C:C + 4, 0:4] = 30.0 * np.eye(4)      # K, head 0
    w[2 * C:, :] = np.eye(C)                # V
    out = O.multi_head_attention(xn, w, np.zeros(3 * C), H)
    np.testing.assert_allclose(out[:, :4], np.eye(4), atol=1e-12)
    np.testing.assert_allclose(out[:, 4:], np.tile(xn[:, 4:].mean(0), (L, 1)), atol=1e-12)


# ---------------------------------------------------------------- block and score (Eqs. 4-6)

def _small(dtype="f32", C=128, heads=2, hidden=512):
    return synth.Workload("t", 2, 13, C, heads, hidden, 1, dtype, True, (0,), (0.7,), "x")


def test_zero_mlp_score_is_norm_of_x_prime():
    wl = _small()
    x = synth.make_input(wl, 5)[0]
    w = synth.make_block_weights(wl, 0, 5, init="full", zero=("w_fc2", "b_fc2"))
    r = O.block_forward(x, w, wl.heads)
    np.testing.assert_allclose(r["score"], np.linalg.norm(r["x_prime"], axis=1), rtol=1e-13)
    np.testing.assert_array_equal(r["x_hat"], r["x_prime"])
    # a constant MLP output c: score = ||c - x'||  (the sign of the subtraction matters
    # only through c; this pins that x' and not x_hat or x is subtracted)
    w2 = dict(w)
    w2["b_fc2"] = np.linspace(-1, 1, wl.C).astype(np.float32)
    r2 = O.block_forward(x, w2, wl.heads)
    np.testing.assert_allclose(r2["score"], np.linalg.norm(w2["b_fc2"] - r2["x_prime"], axis=1),
                               rtol=1e-13)


def test_zero_attention_keeps_residual():
    wl = _small()
    x = synth.make_input(wl, 6)[0]
    w = synth.make_block_weights(wl, 0, 6, init="full", zero=("w_proj", "b_proj", "w_fc2", "b_fc2"))
    r = O.block_forward(x, w, wl.heads)
    np.testing.assert_array_equal(r["x_prime"], x)
    np.testing.assert_allclose(r["score"], np.linalg.norm(x.astype(np.float64), axis=1), rtol=1e-13)
    # b_proj = c shifts x' by c
    w["b_proj"] = np.full(wl.C, 0.5, np.float32)
    np.testing.assert_allclose(O.block_forward(x, w, wl.heads)["x_prime"], x.astype(np.float64) + 0.5,
                               rtol=1e-14)


def test_distances_on_crafted_vectors():
    """Sec. 3.3 distance metrics on vectors whose distances are known by hand."""
    a = np.array([[3.0, 4.0, 0.0], [1.0, 0.0, 0.0], [2.0, 2.0, 0.0], [1.0, 2.0, 0.0], [0.0, 0.0, 0.0]])
    b = np.array([[0.0, 0.0, 0.0], [0.0, 1.0, 0.0], [1.0, 1.0, 0.0], [-2.0, -4.0, 0.0], [0.0, 0.0, 0.0]])
    np.testing.assert_allclose(O.representation_shift(a, b, "l2"), [5.0, 2 ** 0.5, 2 ** 0.5, 45 ** 0.5, 0.0],
                               rtol=1e-15)
    np.testing.assert_allclose(O.representation_shift(a, b, "l1"), [7.0, 2.0, 2.0, 9.0, 0.0], rtol=1e-15)
    # zero vector: distance 1 (reading); orthogonal 1; parallel 0; anti-parallel 2
    np.testing.assert_allclose(O.representation_shift(a, b, "cos"), [1.0, 1.0, 0.0, 2.0, 1.0], atol=1e-15)
    assert O.representation_shift(a, b).tolist() == O.representation_shift(a, b, "l2").tolist()


def test_operation_variants_closed_forms():
    """Sec. 3.3 operation choice with zeroed branches: attention branch zero => the
    attention shift is D(0, x) and the block shift is the size of the MLP output; both
    branches zero => the block shift is D(x, x)."""
    wl = _small()
    x = synth.make_input(wl, 7)[0].astype(np.float64)
    w = synth.make_block_weights(wl, 0, 7, init="full", zero=("w_proj", "b_proj"))
    r2 = O.block_forward(x, w, wl.heads, op="attn", dist="l2")
    np.testing.assert_array_equal(r2["sa"], np.zeros_like(x))
    np.testing.assert_allclose(r2["score"], np.sqrt((x * x).sum(1)), rtol=1e-13)
    np.testing.assert_allclose(O.block_forward(x, w, wl.heads, op="attn", dist="l1")["score"],
                               np.abs(x).sum(1), rtol=1e-13)
    np.testing.assert_allclose(O.block_forward(x, w, wl.heads, op="attn", dist="cos")["score"], 1.0,
                               rtol=0, atol=1e-15)
    # x' = x, x_hat = x + y: the block shift is the size of the MLP output y itself
    rb = O.block_forward(x, w, wl.heads, op="block", dist="l2")
    np.testing.assert_allclose(rb["score"], np.sqrt((rb["mlp"] ** 2).sum(1)), rtol=1e-9)
    np.testing.assert_allclose(O.block_forward(x, w, wl.heads, op="block", dist="l1")["score"],
                               np.abs(rb["mlp"]).sum(1), rtol=1e-9)
    w0 = synth.make_block_weights(wl, 0, 7, init="full", zero=("w_proj", "b_proj", "w_fc2", "b_fc2"))
    np.testing.assert_array_equal(O.block_forward(x, w0, wl.heads, op="block", dist="l2")["score"], 0.0)
    np.testing.assert_array_equal(O.block_forward(x, w0, wl.heads, op="block", dist="l1")["score"], 0.0)
    np.testing.assert_allclose(O.block_forward(x, w0, wl.heads, op="block", dist="cos")["score"], 0.0,
                               atol=1e-15)
    # with every branch live the three operations differ (a dropped-term slip would not)
    wf = synth.make_block_weights(wl, 0, 7, init="full")
    ss = [O.block_forward(x, wf, wl.heads, op=o)["score"] for o in O.SHIFT_OPS]
    assert not np.allclose(ss[0], ss[1]) and not np.allclose(ss[1], ss[2]) and not np.allclose(ss[0], ss[2])


def test_mlp_chain_orientation():
    # fc1 row 2 reads LN channel 1; fc2 row 3 reads hidden unit 2 -> y[:, 3] = GELU(LN(x')[:, 1])
    wl = _small()
    x = synth.make_input(wl, 7)[0]
    w = synth.make_block_weights(wl, 0, 7, init="full")
    for n in ("w_fc1", "b_fc1", "w_fc2", "b_fc2"):
        w[n] = np.zeros_like(w[n])
    w["w_fc1"][2, 1] = 1.0
    w["w_fc2"][3, 2] = 1.0
    r = O.block_forward(x, w, wl.heads)
    ln2 = O.layer_norm(r["x_prime"], w["ln2_g"], w["ln2_b"], wl.ln_eps)
    np.testing.assert_allclose(r["mlp"][:, 3], O.gelu(ln2[:, 1]), rtol=1e-14)
    assert not np.delete(r["mlp"], 3, axis=1).any()


def test_block_fused_equals_materialised_and_permutation_equivariant():
    wl = _small()
    x = synth.make_input(wl, 8)[0]
    w = synth.make_block_weights(wl, 0, 8, init="full")
    a = O.block_forward(x, w, wl.heads)
    b = O.block_forward(x, w, wl.heads, fused_attention=True)
    for key in ("x_hat", "score"):
        np.testing.assert_allclose(a[key], b[key], rtol=1e-12, atol=1e-12)
    perm = np.random.default_rng(9).permutation(x.shape[0])
    c = O.block_forward(x[perm], w, wl.heads)
    np.testing.assert_allclose(c["x_hat"], a["x_hat"][perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(c["score"], a["score"][perm], rtol=1e-12)


# ---------------------------------------------------------------- selection

def _brute_force_topk(s, k, has_cls):
    """The unique k-subset whose every member outranks every non-member."""
    L = len(s)

    def beats(i, j):  # does token i rank above token j?
        if has_cls and (i == 0) != (j == 0):
            return i == 0
        ni, nj = math.isnan(s[i]), math.isnan(s[j])
        if ni != nj:
            return nj
        if not ni and s[i] != s[j]:
            return s[i] > s[j]
        return i < j

    found = []
    for sub in itertools.combinations(range(L), k):
        rest = [j for j in range(L) if j not in sub]
        if all(beats(i, j) for i in sub for j in rest):
            found.append(list(sub))
    assert len(found) == 1
    return found[0]


def test_selection_matches_brute_force_and_argsort():
    rng = np.random.default_rng(10)
    for L in range(1, 9):
        for trial in range(6):
            s = rng.integers(0, 4, size=L).astype(float) if trial % 2 else rng.standard_normal(L)
            if trial == 5 and L > 2:
                s[1] = np.nan
            for k in range(1, L + 1):
                for cls in (False, True):
                    got = O.select_kept(s, k, cls)
                    assert got == _brute_force_topk(list(s), k, cls)
                    assert len(got) == k and got == sorted(set(got))
                    if cls:
                        assert 0 in got
                    if not cls and not np.isnan(s).any():
                        assert got == sorted(np.argsort(-s, kind="stable")[:k].tolist())


def test_selection_special_cases():
    assert O.select_kept([5.0] * 10, 4, False) == [0, 1, 2, 3]          # ties -> lower index
    assert O.select_kept([0.0, 9, 8, 7], 2, True) == [0, 1]              # class token forced
    assert O.select_kept([np.nan, 1, 2, 3], 2, True) == [0, 3]           # forced even if NaN
    assert O.select_kept([1.0, np.nan, 0.5, 2.0], 3, False) == [0, 2, 3]  # NaN dropped first
    assert O.select_kept([1.0, np.inf, 3.0], 1, False) == [1]            # Inf ranks highest
    assert O.select_kept([-1.0, -3.0, -2.0], 2, False) == [0, 2]         # signed scores


# ---------------------------------------------------------------- encoder

def test_identity_blocks_encoder_keeps_largest_norms():
    """All-zero residual branches make every block the identity, so the score is ||x||
    at every prune block and nested selection equals one top-k by row norm."""
    wl = synth.Workload("t", 1, 40, 128, 2, 512, 5, "f32", True, (0, 2, 4), (0.7, 0.6, 0.9), "x")
    x = synth.make_input(wl, 11, spread=True)[0]
    zero = ("w_proj", "b_proj", "w_fc2", "b_fc2")
    blocks = [synth.make_block_weights(wl, b, 11, init="full", zero=zero) for b in range(wl.depth)]
    out, ids = O.encoder_forward(x, blocks, wl.heads, wl.prune_layers, wl.keep_ratios, True)
    _, _, L_final = O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)
    assert L_final == 15 and len(ids) == 15
    expect = O.select_kept(np.linalg.norm(x.astype(np.float64), axis=1), L_final, True)
    assert ids.tolist() == expect
    np.testing.assert_array_equal(out, x[ids])


def test_synth_bf16_rounding():
    a = np.array([1.0, 1.00390625, 1.005859375, -2.0009765625, 3.0e-39], np.float32)
    r = synth.round_to_bf16(a)
    # 1+2^-8 is a tie -> even (1.0); 1+1.5*2^-8 rounds up to 1+2^-7
    np.testing.assert_array_equal(r[:3], np.array([1.0, 1.0, 1.0078125], np.float32))
    assert r[3] == np.float32(-2.0)
    assert (r.view(np.uint32) & 0xFFFF).max() == 0


# ----------------------------------------------------------------------------- around the encoder

def test_patch_embed_is_a_stride_p_convolution():
    """Sec. 3.1 tokenisation: the oracle's patch embedding equals a P x P, stride-P
    convolution (torch's conv2d in float64, a library routine) flattened in raster order,
    frame after frame, with the class token first and the position table added."""
    import torch
    rng = np.random.default_rng(3)
    T, cin, H, W, P, C = 2, 3, 32, 48, 16, 24
    img = rng.standard_normal((T, cin, H, W))
    w = rng.standard_normal((C, cin * P * P))
    b = rng.standard_normal(C)
    cls = rng.standard_normal(C)
    N = T * (H // P) * (W // P)
    pos = rng.standard_normal((N + 1, C))
    got = O.patch_embed(img, w, b, cls, pos, P)
    conv = torch.nn.functional.conv2d(torch.from_numpy(img), torch.from_numpy(w.reshape(C, cin, P, P)),
                                      torch.from_numpy(b), stride=P)          # [T][C][H/P][W/P]
    want = conv.flatten(2).transpose(1, 2).reshape(N, C).numpy()
    np.testing.assert_allclose(got[0], cls + pos[0], rtol=0, atol=0)
    np.testing.assert_allclose(got[1:], want + pos[1:], rtol=1e-12, atol=1e-12)
    # without a class token the table covers the patches only
    got2 = O.patch_embed(img, w, b, None, pos[1:], P)
    np.testing.assert_allclose(got2, want + pos[1:], rtol=1e-12, atol=1e-12)


def test_patch_embed_one_hot_pixel():
    """A one-hot weight row picks pixel (channel 1, row 2, column 5) of every patch: token
    i = pr * (W/P) + pc of frame t holds images[t, 1, pr*P + 2, pc*P + 5]."""
    T, cin, H, W, P = 2, 3, 16, 24, 8
    img = np.arange(T * cin * H * W, dtype=np.float64).reshape(T, cin, H, W)
    w = np.zeros((2, cin * P * P))
    w[1, 1 * P * P + 2 * P + 5] = 1.0
    toks = O.patch_embed(img, w, np.zeros(2), None, np.zeros((T * (H // P) * (W // P), 2)), P)
    gw = W // P
    for t in range(T):
        for pr in range(H // P):
            for pc in range(gw):
                i = t * (H // P) * gw + pr * gw + pc
                assert toks[i, 1] == img[t, 1, pr * P + 2, pc * P + 5]
                assert toks[i, 0] == 0.0


def test_head_pooling_closed_forms():
    """Class-token pooling normalises row 0 only; mean pooling averages the normalised
    rows (not the normalisation of the mean row: the two differ when rows differ in
    scale); a one-hot head reads single features."""
    eps = 1e-6
    C = 4
    g, bt = np.ones(C), np.zeros(C)
    x = np.array([[1.0, -1.0, 0.0, 0.0], [0.0, 0.0, 10.0, -10.0]])
    r = 1.0 / np.sqrt(0.5 + eps)                       # rstd of [1, -1, 0, 0]
    r2 = 1.0 / np.sqrt(50.0 + eps)                     # rstd of [0, 0, 10, -10]
    w = np.eye(C)[[2, 0]]                              # logits = (f[2], f[0]) + b
    hb = np.array([0.5, -0.25])
    f, lg = O.head(x, g, bt, w, hb, "cls", eps)
    np.testing.assert_allclose(f, [r, -r, 0.0, 0.0], rtol=1e-14)
    np.testing.assert_allclose(lg, [0.5, r - 0.25], rtol=1e-14)
    f, lg = O.head(x, g, bt, w, hb, "mean", eps)
    np.testing.assert_allclose(f, [r / 2, -r / 2, 5 * r2, -5 * r2], rtol=1e-14)
    assert abs(f[2] - f[0]) < 1e-5                     # both rows normalise to the same scale
    np.testing.assert_allclose(lg, [5 * r2 + 0.5, r / 2 - 0.25], rtol=1e-14)
    # affine LN parameters apply per channel after normalisation
    f, _ = O.head(x, np.array([2.0, 1.0, 1.0, 1.0]), np.array([0.0, 0.0, 3.0, 0.0]), w, hb, "cls", eps)
    np.testing.assert_allclose(f, [2 * r, -r, 3.0, 0.0], rtol=1e-14)


def test_vit_forward_with_identity_blocks():
    """Identity blocks (zero residual branches) leave the class token's row at cls +
    pos[0], so the features are LN(cls + pos[0]); the kept ids are the top tokens by
    the norm of their embedding."""
    wl = synth.Workload("t", 1, 9, 64, 1, 256, 3, "f32", True, (0, 2), (0.7, 0.8), "x")
    rng = np.random.default_rng(5)
    P, H, W = 8, 16, 32
    img = rng.standard_normal((1, 3, H, W))
    emb = {"w_patch": rng.standard_normal((64, 3 * P * P)) * 0.05, "b_patch": np.zeros(64),
           "cls": np.tile([1.0, -1.0], 32), "pos": np.zeros((9, 64))}
    zero = ("w_proj", "b_proj", "w_fc2", "b_fc2")
    blocks = [synth.make_block_weights(wl, b, 5, init="full", zero=zero) for b in range(wl.depth)]
    hd = {"ln_g": np.ones(64), "ln_b": np.zeros(64), "w_head": np.eye(64)[:8], "b_head": np.zeros(8)}
    feat, logits, ids = O.vit_forward(img, emb, blocks, hd, 1, P, wl.prune_layers, wl.keep_ratios,
                                      True, "cls")
    np.testing.assert_allclose(feat, np.tile([1.0, -1.0], 32) / np.sqrt(1 + 1e-6), rtol=1e-12)
    np.testing.assert_allclose(logits, feat[:8], rtol=0, atol=0)
    toks = O.patch_embed(img, emb["w_patch"], emb["b_patch"], emb["cls"], emb["pos"], P)
    k1 = O.keep_count(0.7, 9)
    k2 = O.keep_count(0.8, k1)
    assert ids.tolist() == O.select_kept(np.linalg.norm(toks, axis=1), k2, True)


# ----------------------------------------------------------------------------- Eq. (2) / Eq. (3)

def test_attention_map_scores_closed_forms():
    """Eq. (2) and Eq. (3) on maps whose softmax has a closed form: zero queries give
    uniform rows (every score 1/L); one head with two keys whose logits differ by t has
    rows (sigma(t), 1 - sigma(t)); each Eq. (3) score vector sums to 1 (mean of rows that
    each sum to 1); heads are averaged."""
    L, C, heads = 5, 128, 2
    xn = np.random.default_rng(0).standard_normal((L, C))
    w = np.zeros((3 * C, C))
    w[C:2 * C] = np.random.default_rng(1).standard_normal((C, C))   # keys only: Q = 0
    maps = O.attention_maps(xn, w, np.zeros(3 * C), heads)
    assert maps.shape == (heads, L, L)
    for kind in ("cls", "mean"):
        np.testing.assert_allclose(O.attention_map_score(maps, kind), np.full(L, 1.0 / L), rtol=1e-14)
    # hand-built maps: head 0 rows (a, 1-a) with a = sigma(t); head 1 uniform
    t = 0.7
    a = 1.0 / (1.0 + math.exp(-t))
    m = np.array([[[a, 1 - a], [1 - a, a]], [[0.5, 0.5], [0.5, 0.5]]])
    np.testing.assert_allclose(O.attention_map_score(m, "cls"), [(a + 0.5) / 2, (1 - a + 0.5) / 2], rtol=1e-14)
    np.testing.assert_allclose(O.attention_map_score(m, "mean"), [0.5, 0.5], rtol=1e-14)
    # a real map from logits: query 0 attends by exp(q.k / 8); Eq. (3) sums to 1
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 64))
    wq = rng.standard_normal((192, 64)) * 0.3
    maps = O.attention_maps(x, wq, np.zeros(192), 1)
    q, k = x @ wq[:64].T, x @ wq[64:128].T
    e = np.exp(q[0] @ k.T / 8.0)
    np.testing.assert_allclose(O.attention_map_score(maps, "cls"), e / e.sum(), rtol=1e-12)
    mean = O.attention_map_score(maps, "mean")
    assert abs(mean.sum() - 1.0) < 1e-12
    np.testing.assert_allclose(mean[3], np.mean([np.exp(q[i] @ k[3] / 8) / np.exp(q[i] @ k.T / 8).sum()
                                                  for i in range(7)]), rtol=1e-12)


def test_block_map_scores_use_the_blocks_own_map():
    """The block's map score is computed from LN1(x) through W_qkv (the attention the block
    runs); it does not depend on the projection or the MLP."""
    wl = synth.Workload("t", 1, 9, 128, 2, 512, 1, "f32", True, (0,), (0.7,), "x")
    x = synth.make_input(wl, 3)[0]
    w = synth.make_block_weights(wl, 0, 3, init="full")
    w2 = dict(w, w_proj=w["w_proj"] * 3.0, w_fc2=w["w_fc1"].T.copy() * 0.0 + 0.01)
    for op, kind in (("map_cls", "cls"), ("map_mean", "mean")):
        r = O.block_forward(x, w, wl.heads, op=op)
        xn = O.layer_norm(x, w["ln1_g"], w["ln1_b"], 1e-6)
        want = O.attention_map_score(O.attention_maps(xn, w["w_qkv"], w["b_qkv"], wl.heads), kind)
        np.testing.assert_allclose(r["score"], want, rtol=1e-14)
        np.testing.assert_allclose(O.block_forward(x, w2, wl.heads, op=op)["score"], want, rtol=1e-14)
        # the block output is the method's
        np.testing.assert_array_equal(r["x_hat"], O.block_forward(x, w, wl.heads)["x_hat"])

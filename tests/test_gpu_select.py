"""GPU parity of the selection kernels through the C ABI: rs_topk_gather (bit-exact
indices and rows against the oracle's selection) and rs_score (Eq. (4), L2)."""
import numpy as np
import pytest

from oracle import rs_oracle as O
import synth

pytestmark = pytest.mark.gpu

# (B, L, k, has_cls, score kind): every stage shape of the four encoder workloads, plus
# degenerate and maximum sizes
STAGES = [
    (256, 197, 138, True), (256, 138, 97, True), (256, 97, 68, True),
    (128, 197, 128, True), (128, 128, 83, True), (128, 83, 54, True),
    (8, 1568, 784, False), (8, 784, 392, False), (8, 392, 196, False),
    (4, 1568, 784, False), (4, 784, 392, False), (4, 392, 196, False), (4, 196, 98, False),
    (2, 197, 138, True),
]
EDGES = [
    (1, 1, 1, True), (1, 1, 1, False), (3, 5, 5, False), (3, 5, 5, True), (2, 7, 1, True),
    (2, 7, 1, False), (5, 1000, 1, False), (2, 16384, 1, False), (2, 16384, 16384, True),
    (2, 16384, 8191, False), (3, 1025, 513, True), (1, 2352, 1882, False),
]


def _run(B, L, k, cls, kind, seed, C=64, inject=True):
    import torch
    import vit_token_pruning_amd as rs
    s = synth.make_scores(B, L, seed, kind)
    if inject and L >= 6:
        s[0, 3] = np.nan
        s[-1, 1] = np.inf
        s[-1, 2] = -0.0
        s[-1, 4] = 0.0
    x = synth.round_to_bf16(np.random.default_rng(seed).standard_normal((B, L, C)).astype(np.float32))
    sd = torch.from_numpy(s).cuda()
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    kept, xk = rs.topk_gather(sd, xd, k, cls)
    torch.cuda.synchronize()
    kept = kept.cpu().numpy()
    xk = xk.float().cpu().numpy()
    for b in range(B):
        want = O.select_kept(s[b], k, cls)
        assert kept[b].tolist() == want, f"sample {b}"
        np.testing.assert_array_equal(xk[b], x[b][want])


@pytest.mark.parametrize("B,L,k,cls", STAGES)
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_topk_gather_stage_shapes(B, L, k, cls, kind):
    _run(B, L, k, cls, kind, seed=L * 7 + k)


@pytest.mark.parametrize("B,L,k,cls", EDGES)
@pytest.mark.parametrize("kind", ["normal", "ties", "signed"])
def test_topk_gather_edges(B, L, k, cls, kind):
    _run(B, L, k, cls, kind, seed=L + 3 * k + B)


# The kept rows are copied inside the top-k launch by ceil(128 / B) (at most 64) workgroups
# per sample, each copying a contiguous share; L <= 256 takes the single-wave selection,
# longer L the 1024-thread radix select.  Row widths of 3 to 1032 16-byte units (over 1024
# units a row is copied by all threads in turn); shares of zero rows when k < the split.
FUSED = [(64, 1568, 784, False, 256), (40, 2000, 37, True, 64), (32, 1025, 1, True, 1024),
         (33, 300, 299, False, 8), (32, 1024, 1024, True, 384), (48, 16384, 9000, False, 8),
         (32, 256, 255, False, 8192), (36, 256, 1, True, 16), (32, 257, 128, True, 24),
         (32, 40, 20, False, 8256), (1, 1568, 700, False, 8256), (3, 300, 299, True, 8192),
         (7, 97, 5, True, 384), (2, 2352, 1882, False, 768), (129, 197, 138, True, 384)]


@pytest.mark.parametrize("B,L,k,cls,C", FUSED)
def test_topk_gather_fused_copy(B, L, k, cls, C):
    _run(B, L, k, cls, "ties", seed=B + L + k, C=C)


def test_topk_select_only_and_fp32_rows():
    import torch
    import vit_token_pruning_amd as rs
    s = synth.make_scores(3, 300, 5, "ties")
    sd = torch.from_numpy(s).cuda()
    kept, xk = rs.topk_gather(sd, None, 100, False)
    assert xk is None
    for b in range(3):
        assert kept[b].cpu().tolist() == O.select_kept(s[b], 100, False)
    x = np.random.default_rng(1).standard_normal((3, 300, 192)).astype(np.float32)
    kept, xk = rs.topk_gather(sd, torch.from_numpy(x).cuda(), 100, True)
    for b in range(3):
        want = O.select_kept(s[b], 100, True)
        np.testing.assert_array_equal(xk[b].cpu().numpy(), x[b][want])


@pytest.mark.parametrize("dt,B,L,C", [("bf16", 256, 197, 384), ("bf16", 8, 1568, 768),
                                      ("f32", 2, 197, 192), ("bf16", 1, 1, 8), ("f32", 3, 77, 1024)])
def test_score_matches_oracle(dt, B, L, C):
    import torch
    import vit_token_pruning_amd as rs
    rng = np.random.default_rng(B + L + C)
    a = rng.standard_normal((B, L, C)).astype(np.float32)
    b = (a + 0.3 * rng.standard_normal((B, L, C))).astype(np.float32)
    if dt == "bf16":
        a, b = synth.round_to_bf16(a), synth.round_to_bf16(b)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    s = rs.score(torch.from_numpy(a).cuda().to(tdt), torch.from_numpy(b).cuda().to(tdt))
    got = s.cpu().numpy().astype(np.float64)
    want = O.representation_shift(a, b)
    rel = np.abs(got - want) / want
    # bar: 1e-2 relative; the arithmetic (exact inputs, fp32 sum of <= 1024 squares) is
    # good to ~C * 2^-24, so anything above 1e-4 would indicate a defect
    assert rel.max() <= 1e-4
    assert rs.score(torch.zeros(2, 3, 64, device="cuda"), torch.zeros(2, 3, 64, device="cuda")).abs().max() == 0


# Boundaries of the keys-per-thread instantiations of the selection (1, 2, 4, 8 and 32 keys
# per thread: L up to 512, 1024, 2048, 4096 and 16384) and score sets that stress the radix
# passes: every competing score equal (no bit to resolve), two distinct values, scores spread
# over the whole float range (keys differing in the top bit), and many NaNs.
BOUNDS = [(3, 256, 100, True), (3, 257, 100, False), (2, 512, 511, True), (2, 513, 2, False),
          (2, 1024, 1023, False), (2, 1025, 700, True), (2, 2048, 1024, False),
          (2, 2049, 1024, True), (4, 1568, 1, True), (4, 1568, 1568, False),
          (2, 4096, 2048, False), (2, 4097, 4000, True), (1, 8193, 1, False), (1, 12000, 11999, True)]


@pytest.mark.parametrize("B,L,k,cls", BOUNDS)
@pytest.mark.parametrize("kind", ["normal", "ties", "signed"])
def test_topk_gather_wave_boundaries(B, L, k, cls, kind):
    _run(B, L, k, cls, kind, seed=5 * L + k + B)


@pytest.mark.parametrize("L,k,cls", [(197, 138, True), (1568, 784, False), (700, 350, True)])
@pytest.mark.parametrize("pattern", ["equal", "two", "wide", "nans"])
def test_topk_gather_degenerate_scores(L, k, cls, pattern):
    import torch
    import vit_token_pruning_amd as rs
    B = 3
    rng = np.random.default_rng([L, k, len(pattern)])
    if pattern == "equal":
        s = np.full((B, L), 7.25, np.float32)
    elif pattern == "two":
        s = np.where(rng.random((B, L)) < 0.5, 3.0, 5.0).astype(np.float32)
    elif pattern == "wide":
        s = (np.sign(rng.standard_normal((B, L))) *
             np.exp2(rng.uniform(-120, 120, (B, L)))).astype(np.float32)
    else:
        s = rng.standard_normal((B, L)).astype(np.float32)
        s[rng.random((B, L)) < 0.3] = np.nan
    x = synth.round_to_bf16(rng.standard_normal((B, L, 64)).astype(np.float32))
    kept, xk = rs.topk_gather(torch.from_numpy(s).cuda(), torch.from_numpy(x).cuda().to(torch.bfloat16), k, cls)
    torch.cuda.synchronize()
    kept, xk = kept.cpu().numpy(), xk.float().cpu().numpy()
    for b in range(B):
        want = O.select_kept(s[b], k, cls)
        assert kept[b].tolist() == want, f"sample {b}"
        np.testing.assert_array_equal(xk[b], x[b][want])

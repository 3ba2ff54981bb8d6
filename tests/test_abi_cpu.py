"""CPU-only checks of the C ABI: the library loads, exports every symbol include/rs.h
declares, and rejects bad arguments synchronously, before any HIP call (so these
run without a GPU).  No compute call is made here."""
import ctypes
import os

import pytest

from oracle import rs_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def N():
    from vit_token_pruning_amd import _native
    if not os.path.exists(_native.LIB_PATH):
        from vit_token_pruning_amd import build
        build.build()
    _native.lib()
    return _native


def test_every_declared_symbol_is_exported(N):
    names = N.declared_symbols()
    assert {"rs_block_forward", "rs_score", "rs_topk_gather", "rs_encoder_forward"} <= set(names)
    for n in names:
        assert hasattr(N.lib(), n), n


def _desc(N, C=384, heads=6, hidden=1536, dtype=1, has_cls=1, eps=1e-6, op=0, dist=0, amap=0):
    return N.ModelDesc(C, heads, hidden, eps, dtype, has_cls, op, dist, amap)


FAKE = 1 << 20  # an aligned non-null address; never dereferenced (validation fails first)


def _weights(N, p=FAKE):
    return N.BlockWeights(*([p] * 12))


def _block_call(N, desc=None, w=None, x=FAKE, B=2, L=197, k=138, y=FAKE, s=FAKE, kept=FAKE,
                yk=FAKE, ws=FAKE, ws_bytes=None):
    lib = N.lib()
    desc = desc if desc is not None else _desc(N)
    w = w if w is not None else _weights(N)
    if ws_bytes is None:
        ws_bytes = lib.rs_workspace_bytes(ctypes.byref(desc), 1, B, L) if desc.C > 0 else 0
    return lib.rs_block_forward(ctypes.byref(desc), ctypes.byref(w), x, B, L, k, y, s, kept, yk,
                                ws, ws_bytes, None)


def test_block_forward_validation(N):
    lib = N.lib()
    E_ARG, E_UNS, E_WS = N.RS_ERR_INVALID_ARG, N.RS_ERR_UNSUPPORTED, N.RS_ERR_WORKSPACE
    cases = [
        (dict(desc=_desc(N, dtype=7)), E_ARG),
        (dict(desc=_desc(N, C=384, heads=4)), E_UNS),          # head dim != 64
        (dict(desc=_desc(N, C=200, heads=3)), E_UNS),          # C % 64
        (dict(desc=_desc(N, hidden=1000)), E_UNS),
        (dict(desc=_desc(N, eps=0.0)), E_ARG),
        (dict(desc=_desc(N, has_cls=2)), E_ARG),
        (dict(desc=_desc(N, op=5)), E_ARG),                     # unknown score operation
        (dict(desc=_desc(N, op=3, has_cls=0)), E_ARG),          # Eq. (2) needs a class token
        (dict(desc=_desc(N, amap=2)), E_ARG),
        (dict(desc=_desc(N, op=-1)), E_ARG),
        (dict(desc=_desc(N, dist=3)), E_ARG),                   # unknown distance
        (dict(k=0), E_ARG),
        (dict(k=198), E_ARG),
        (dict(L=0, k=1), E_ARG),
        (dict(L=20000, k=5), E_UNS),
        (dict(x=None), E_ARG),
        (dict(x=FAKE + 4), E_ARG),                              # misaligned
        (dict(kept=None), E_ARG),
        (dict(yk=None), E_ARG),
        (dict(w=_weights(N, 0)), E_ARG),
        (dict(ws=FAKE + 16), E_ARG),                            # workspace not 256-aligned
        (dict(ws_bytes=1024), E_WS),
    ]
    for kw, want in cases:
        got = _block_call(N, **kw)
        assert got == want, (kw, got, lib.rs_last_error())
        assert lib.rs_last_error().decode()


def test_score_and_topk_validation(N):
    lib = N.lib()
    assert lib.rs_score(FAKE, FAKE, 2, 10, 100, 1, FAKE, None) == N.RS_ERR_UNSUPPORTED  # C % 8
    assert lib.rs_score(None, FAKE, 2, 10, 64, 1, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_score(FAKE, FAKE, 2, 10, 64, 5, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_score_dist(FAKE, FAKE, 2, 10, 64, 1, 3, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_score_dist(FAKE, FAKE, 2, 10, 100, 1, 1, FAKE, None) == N.RS_ERR_UNSUPPORTED
    assert lib.rs_score_dist(FAKE, FAKE, 2, 10, 64, 1, 2, None, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_topk_gather(FAKE, FAKE, 2, 10, 64, 1, 0, 1, FAKE, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_topk_gather(FAKE, FAKE, 2, 10, 64, 1, 11, 1, FAKE, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_topk_gather(FAKE, FAKE, 2, 10, 64, 1, 5, 3, FAKE, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_topk_gather(None, FAKE, 2, 10, 64, 1, 5, 1, FAKE, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_topk_gather(FAKE, FAKE, 2, 10, 3, 1, 5, 1, FAKE, FAKE, None) == N.RS_ERR_UNSUPPORTED
    assert lib.rs_topk_gather(FAKE, FAKE, 2, 10, 64, 1, 5, 1, FAKE, FAKE + 8, None) == N.RS_ERR_INVALID_ARG


def test_encoder_schedule_matches_oracle(N):
    import synth
    lib = N.lib()
    for wl in synth.WORKLOADS.values():
        out = ctypes.c_int()
        st = lib.rs_encoder_out_len(wl.depth, wl.L, N.int_array(wl.prune_layers),
                                    N.dbl_array(wl.keep_ratios), len(wl.prune_layers), ctypes.byref(out))
        assert st == N.RS_OK
        assert out.value == O.schedule(wl.depth, wl.L, wl.prune_layers, wl.keep_ratios)[2]
    # round-half-up cases evaluated in double on both sides
    for r, L in [(0.5, 3), (0.9, 1905), (0.7, 197), (0.65, 83), (0.1, 5), (1.0, 1)]:
        out = ctypes.c_int()
        assert lib.rs_encoder_out_len(1, L, N.int_array([0]), N.dbl_array([r]), 1,
                                      ctypes.byref(out)) == N.RS_OK
        assert out.value == O.keep_count(r, L)


def test_encoder_validation(N):
    lib = N.lib()
    out = ctypes.c_int()

    def ol(depth, L, pl, kr):
        return lib.rs_encoder_out_len(depth, L, N.int_array(pl), N.dbl_array(kr), len(pl), ctypes.byref(out))

    assert ol(12, 197, [3, 3], [0.7, 0.7]) == N.RS_ERR_INVALID_ARG      # not strictly ascending
    assert ol(12, 197, [6, 3], [0.7, 0.7]) == N.RS_ERR_INVALID_ARG
    assert ol(12, 197, [12], [0.7]) == N.RS_ERR_INVALID_ARG             # >= depth
    assert ol(12, 197, [-1], [0.7]) == N.RS_ERR_INVALID_ARG
    assert ol(12, 197, [1], [0.0]) == N.RS_ERR_INVALID_ARG
    assert ol(12, 197, [1], [1.5]) == N.RS_ERR_INVALID_ARG
    assert ol(12, 197, [1], [float("nan")]) == N.RS_ERR_INVALID_ARG
    assert ol(12, 4, [1], [0.1]) == N.RS_ERR_INVALID_ARG                # keeps 0 tokens
    assert ol(0, 197, [], []) == N.RS_ERR_INVALID_ARG
    d = _desc(N)
    blocks = (N.BlockWeights * 12)(*[_weights(N) for _ in range(12)])
    ws = lib.rs_workspace_bytes(ctypes.byref(d), 12, 4, 197)
    assert ws > 0
    st = lib.rs_encoder_forward(ctypes.byref(d), blocks, 12, FAKE, 4, 197, N.int_array([3, 6, 9]),
                                N.dbl_array([0.7] * 3), 3, FAKE, FAKE, FAKE, ws // 4, None)
    assert st == N.RS_ERR_WORKSPACE
    blocks[5] = _weights(N, 0)
    st = lib.rs_encoder_forward(ctypes.byref(d), blocks, 12, FAKE, 4, 197, N.int_array([3, 6, 9]),
                                N.dbl_array([0.7] * 3), 3, FAKE, FAKE, FAKE, ws, None)
    assert st == N.RS_ERR_INVALID_ARG and b"block 5" in lib.rs_last_error()


def test_workspace_query(N):
    lib = N.lib()
    assert lib.rs_workspace_bytes(None, 1, 2, 197) == 0
    bad = _desc(N, C=100)
    assert lib.rs_workspace_bytes(ctypes.byref(bad), 1, 2, 197) == 0
    d = _desc(N)
    a = lib.rs_workspace_bytes(ctypes.byref(d), 1, 256, 197)
    b = lib.rs_workspace_bytes(ctypes.byref(d), 12, 256, 197)
    # activations for one block plus the per-call weights of every block: W_qkv (folded,
    # or packed for the weight-streaming kernel), and for bf16 at C <= 384 the fused MLP
    # kernel's packed W1 and W2 and the packed W_proj
    fold = 3 * 384 * 384 * 2 + 2 * 384 * 1536 * 2 + 384 * 384 * 2
    assert a % 256 == 0 and a > 256 * 197 * 384 * 2 * 8
    assert b - a >= 11 * fold and b - a < 11 * (fold + 64 * 1024)
    # stored attention maps: B * H * L * pad8(L) elements; Eq. (3) column sums per 64 queries
    m = lib.rs_workspace_bytes(ctypes.byref(_desc(N, amap=1)), 1, 256, 197)
    assert 256 * 6 * 197 * 200 * 2 <= m - a < 256 * 6 * 197 * 200 * 2 + 4096
    m = lib.rs_workspace_bytes(ctypes.byref(_desc(N, op=4)), 1, 256, 197)
    assert 256 * 6 * 4 * 197 * 4 <= m - a < 256 * 6 * 4 * 197 * 4 + 4096
    m = lib.rs_workspace_bytes(ctypes.byref(_desc(N, op=3)), 1, 256, 197)
    assert 256 * 6 * 197 * 4 <= m - a < 256 * 6 * 197 * 4 + 4096
    # the cosine distance keeps three partial sums per 64-column slice instead of one
    for op in (0, 1, 2):
        c = _desc(N, op=op, dist=2)
        l1 = _desc(N, op=op, dist=1)
        assert lib.rs_workspace_bytes(ctypes.byref(l1), 1, 256, 197) == a
        extra = lib.rs_workspace_bytes(ctypes.byref(c), 1, 256, 197) - a
        assert 256 * 197 * 6 * 2 * 4 <= extra < 256 * 197 * 6 * 2 * 4 + 4096   # 6 slices of 64


def test_set_max_lanes(N):
    lib = N.lib()
    assert lib.rs_set_max_lanes(0) == N.RS_ERR_INVALID_ARG
    assert lib.rs_set_max_lanes(5) == N.RS_ERR_INVALID_ARG
    for n in (1, 3, 4, 2):
        assert lib.rs_set_max_lanes(n) == N.RS_OK


def test_timing_session_without_launches(N):
    lib = N.lib()
    assert lib.rs_timing_begin(99) == N.RS_ERR_INVALID_ARG
    assert lib.rs_timing_end(None, None, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_timing_begin(4) == N.RS_OK
    assert lib.rs_timing_begin(4) == N.RS_ERR_INVALID_ARG
    ms, n, work = ctypes.c_float(1), ctypes.c_int(1), ctypes.c_double(1)
    assert lib.rs_timing_end(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(work)) == N.RS_OK
    assert ms.value == 0 and n.value == 0 and work.value == 0


def test_product_path_does_not_touch_the_oracle():
    """The package and the HIP sources never name the oracle or the input generators."""
    pkg = os.path.join(ROOT, "vit_token_pruning_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.lower(), f
                assert "import synth" not in text and "from synth" not in text, f


def test_patch_embed_head_and_forward_validation(N):
    lib = N.lib()
    E_ARG, E_UNS = N.RS_ERR_INVALID_ARG, N.RS_ERR_UNSUPPORTED
    d = _desc(N)
    emb = N.EmbedWeights(FAKE, FAKE, FAKE, FAKE)

    def pe(img, e=emb, desc=d, B=2, images=FAKE, tokens=FAKE):
        return lib.rs_patch_embed(ctypes.byref(desc), ctypes.byref(img) if img is not None else None,
                                  ctypes.byref(e), images, B, tokens, None)

    good = N.ImageDesc(1, 3, 224, 224, 16)
    assert pe(None) == E_ARG
    assert pe(N.ImageDesc(1, 3, 224, 224, 12)) == E_UNS                 # patch not 8/16/32
    assert pe(N.ImageDesc(1, 3, 224, 200, 16)) == E_ARG                 # width % patch
    assert pe(N.ImageDesc(0, 3, 224, 224, 16)) == E_ARG
    assert pe(N.ImageDesc(1, 0, 224, 224, 16)) == E_ARG
    assert pe(N.ImageDesc(1000, 3, 224, 224, 16)) == E_UNS              # > RS_MAX_TOKENS
    assert pe(good, e=N.EmbedWeights(FAKE, FAKE, None, FAKE)) == E_ARG  # class token missing
    assert pe(good, B=0) == E_ARG
    assert pe(good, images=None) == E_ARG
    assert pe(good, tokens=FAKE + 8) == E_ARG
    assert pe(good, desc=_desc(N, op=5)) == E_ARG
    nocls = _desc(N, has_cls=0)
    hw = N.HeadWeights(FAKE, FAKE, FAKE, FAKE, 1000, N.RS_POOL_CLS)

    def hd(h, desc=d, B=2, L=68, x=FAKE, f=FAKE, lg=FAKE, ws=FAKE, ws_bytes=1 << 20):
        return lib.rs_head(ctypes.byref(desc), ctypes.byref(h), x, B, L, f, lg, ws, ws_bytes, None)

    assert hd(N.HeadWeights(FAKE, FAKE, FAKE, FAKE, 1001, N.RS_POOL_CLS)) == E_UNS   # n_out % 8
    assert hd(N.HeadWeights(FAKE, FAKE, FAKE, FAKE, 0, N.RS_POOL_CLS)) == E_UNS
    assert hd(N.HeadWeights(FAKE, FAKE, FAKE, FAKE, 1000, 2)) == E_ARG               # pool
    assert hd(hw, desc=nocls) == E_ARG                                               # no class token
    assert hd(N.HeadWeights(FAKE, None, FAKE, FAKE, 1000, N.RS_POOL_CLS)) == E_ARG
    assert hd(hw, f=None) == E_ARG
    assert hd(hw, L=0) == E_ARG
    assert hd(hw, ws=FAKE + 64) == E_ARG                                             # alignment
    need = lib.rs_head_workspace_bytes(2, 68, 384)
    assert need == 3 * 2 * 384 * 4 and lib.rs_head_workspace_bytes(2, 68, 100) == 0  # 3 row blocks
    assert hd(hw, ws_bytes=need - 1) == N.RS_ERR_WORKSPACE
    # whole forward: workspace query and checks before anything is enqueued
    n1 = lib.rs_vit_workspace_bytes(ctypes.byref(d), ctypes.byref(good), 12, 256)
    assert n1 > 0
    assert lib.rs_vit_workspace_bytes(ctypes.byref(d), ctypes.byref(N.ImageDesc(1, 3, 224, 224, 12)), 12, 256) == 0
    enc_ws = lib.rs_workspace_bytes(ctypes.byref(d), 12, 256, 197)
    assert n1 > enc_ws + 2 * 256 * 197 * 384 * 2                          # tokens + encoder output
    blocks = (N.BlockWeights * 12)(*[_weights(N) for _ in range(12)])
    pl, kr = N.int_array([3, 6, 9]), N.dbl_array([0.7] * 3)

    def fw(ws_bytes=n1, img=good, h=hw, sched=(pl, kr, 3)):
        return lib.rs_vit_forward(ctypes.byref(d), ctypes.byref(img), ctypes.byref(emb), blocks, 12,
                                  ctypes.byref(h), FAKE, 256, sched[0], sched[1], sched[2], FAKE,
                                  FAKE, None, FAKE, ws_bytes, None)

    assert fw(ws_bytes=n1 // 2) == N.RS_ERR_WORKSPACE
    assert fw(sched=(N.int_array([3, 3]), N.dbl_array([0.7, 0.7]), 2)) == E_ARG
    assert fw(h=N.HeadWeights(FAKE, FAKE, FAKE, FAKE, 12, N.RS_POOL_CLS)) == E_UNS
    assert fw(img=N.ImageDesc(1, 3, 224, 224, 12)) == E_UNS


def test_attention_noalloc_validation(N):
    """rs_attention_noalloc validates like rs_attention and rejects, before any HIP call, a
    score whose sums exceed the library's fixed scratch (16 MiB)."""
    lib = N.lib()
    d = _desc(N, C=768, heads=12, hidden=3072, has_cls=0)
    # Eq. (3) column sums of 20 clips x 2352 tokens x 12 heads x 37 query blocks: ~84 MB
    st = lib.rs_attention_noalloc(ctypes.byref(d), FAKE, 20, 2352, FAKE, None, None, FAKE, None)
    assert st == N.RS_ERR_UNSUPPORTED
    assert b"scratch" in lib.rs_last_error()
    assert lib.rs_attention_workspace_bytes(ctypes.byref(d), 20, 2352) > (16 << 20)
    # the usual argument checks come first
    assert lib.rs_attention_noalloc(ctypes.byref(d), None, 2, 197, FAKE, None, None, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_attention_noalloc(ctypes.byref(d), FAKE, 2, 197, FAKE + 4, None, None, None, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_attention_noalloc(ctypes.byref(d), FAKE, 0, 197, FAKE, None, None, None, None) == N.RS_ERR_INVALID_ARG


def test_probe_validation(N):
    """rs_probe_throughput rejects, before any HIP call, a mode outside 0..6, an empty grid or
    iteration count, and a null sink."""
    lib = N.lib()
    assert lib.rs_probe_throughput(7, 1024, 10, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert b"mode" in lib.rs_last_error()
    assert lib.rs_probe_throughput(-1, 1024, 10, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_probe_throughput(0, 0, 10, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_probe_throughput(0, 1024, 0, FAKE, None) == N.RS_ERR_INVALID_ARG
    assert lib.rs_probe_throughput(2, 1024, 10, None, None) == N.RS_ERR_INVALID_ARG

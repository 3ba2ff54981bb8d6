"""rs_attention_noalloc (the entry point that allocates nothing; its score sums live in the
library's fixed per-device scratch array) against rs_attention with a caller workspace:
same kernels, same inputs, so every output must be bit-identical.  Two calls in a row on
one stream, the second with a smaller input, each also compared with the oracle's
attention-map scores (Eq. (2) and Eq. (3) of the arXiv page, Sec. 3.1, averaged over heads)."""
import ctypes

import numpy as np
import pytest

from oracle import rs_oracle as O
import synth
from rs_testutil import spec_of, to_dev, to_host

pytestmark = pytest.mark.gpu


def _run(fn_name, spec, qkv, want_map, ws=None):
    import torch
    import vit_token_pruning_amd as rs
    from vit_token_pruning_amd import _native as N
    B, L, _ = qkv.shape
    dev = qkv.device
    out = torch.full((B, L, spec.C), float("nan"), dtype=spec.dtype, device=dev)
    lpad = (L + 7) // 8 * 8
    amap = torch.full((B, spec.heads, L, lpad), float("nan"), dtype=spec.dtype, device=dev) if want_map else None
    sc = torch.full((B, L), float("nan"), dtype=torch.float32, device=dev)
    sm = torch.full((B, L), float("nan"), dtype=torch.float32, device=dev)
    d = spec.desc()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = rs.lib()
    if fn_name == "rs_attention_noalloc":
        st = lib.rs_attention_noalloc(ctypes.byref(d), qkv.data_ptr(), B, L, out.data_ptr(),
                                      amap.data_ptr() if want_map else None, sc.data_ptr(),
                                      sm.data_ptr(), stream)
    else:
        st = lib.rs_attention(ctypes.byref(d), qkv.data_ptr(), B, L, out.data_ptr(),
                              amap.data_ptr() if want_map else None, sc.data_ptr(), sm.data_ptr(),
                              ws.data_ptr(), ws.numel(), stream)
    N.check(fn_name, st)
    return out, amap, sc, sm


@pytest.mark.parametrize("name,shapes", [("deit_s", [(8, 197), (3, 68)]),
                                         ("umt_b", [(2, 1568), (1, 392)]),
                                         ("deit_t_block", [(2, 197), (1, 65)])])
def test_noalloc_attention_matches_workspace_entry_point(name, shapes):
    import torch
    import vit_token_pruning_amd as rs
    wl = synth.WORKLOADS[name]
    spec = spec_of(wl)
    for i, (B, L) in enumerate(shapes):
        print(f"case {name} B{B} L{L} call {i}", flush=True)
        rng = np.random.default_rng([31, i, L])
        qkv_np = rng.standard_normal((B, L, 3 * wl.C)).astype(np.float32)
        if wl.dtype == "bf16":
            qkv_np = synth.round_to_bf16(qkv_np)
        qkv = to_dev(qkv_np, wl.dtype)
        want_map = L <= 256
        a = _run("rs_attention_noalloc", spec, qkv, want_map)
        d = spec.desc()
        nws = int(rs.lib().rs_attention_workspace_bytes(ctypes.byref(d), B, L))
        assert 0 < nws <= 16 << 20
        ws = torch.empty(nws, dtype=torch.uint8, device="cuda")
        b = _run("rs_attention", spec, qkv, want_map, ws)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            if x is not None:
                assert torch.equal(x, y), "no-alloc output differs from the workspace entry point"
        # and against the oracle's map scores (fp64, per sample)
        sc, sm = a[2].cpu().numpy(), a[3].cpu().numpy()
        tol = 1e-3 if wl.dtype == "bf16" else 1e-5
        C = wl.C
        for s in range(B):
            maps = np.stack([O.softmax_rows(qkv_np[s, :, h * 64:(h + 1) * 64].astype(np.float64)
                                            @ qkv_np[s, :, C + h * 64:C + (h + 1) * 64].astype(np.float64).T
                                            / 8.0) for h in range(wl.heads)])
            want_cls = O.attention_map_score(maps, "cls")
            want_mean = O.attention_map_score(maps, "mean")
            assert np.abs(sc[s] - want_cls).max() <= tol * max(1.0, np.abs(want_cls).max())
            assert np.abs(sm[s] - want_mean).max() <= tol * max(1.0, np.abs(want_mean).max())


def test_noalloc_fused_path_needs_no_scratch():
    """Without scores the fused kernel runs and the scratch is not touched."""
    import torch
    import vit_token_pruning_amd as rs
    from vit_token_pruning_amd import _native as N
    wl = synth.WORKLOADS["deit_s"]
    spec = spec_of(wl)
    B, L = 2, 197
    qkv = to_dev(synth.round_to_bf16(np.random.default_rng(5).standard_normal((B, L, 3 * wl.C)).astype(np.float32)),
                 "bf16")
    out = torch.empty(B, L, wl.C, dtype=torch.bfloat16, device="cuda")
    d = spec.desc()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    N.check("rs_attention_noalloc", rs.lib().rs_attention_noalloc(
        ctypes.byref(d), qkv.data_ptr(), B, L, out.data_ptr(), None, None, None, stream))
    ref, _, _, _ = rs.attention(spec, qkv)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)

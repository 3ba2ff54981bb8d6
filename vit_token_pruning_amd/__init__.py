"""Representation Shift token pruning on MI355X: torch-facing wrappers of librs.so.

Every function takes CUDA (HIP) torch tensors, checks shapes/dtypes/devices, and
passes raw pointers plus the current stream to the C ABI of include/rs.h.  Outputs are
allocated with torch.  No step of the method runs in Python or on the CPU here.
"""
from __future__ import annotations

import ctypes
from typing import Dict, List, Optional, Sequence

import torch

from . import _native as N
from ._native import BLOCK_FIELDS, KERNELS, RSError, lib  # noqa: F401

__all__ = ["ModelSpec", "block_forward", "score", "topk_gather", "encoder_forward",
           "encoder_out_len", "workspace_bytes", "Encoder", "KernelTimer", "RSError", "lib",
           "set_max_lanes", "get_max_lanes", "ImageSpec", "patch_embed", "head", "ViT", "vit_forward", "attention"]

_DT = {torch.float32: N.RS_F32, torch.bfloat16: N.RS_BF16}
# representation shift variants of the ablations and the attention-map baselines
# (rs_shift_op, rs_dist of include/rs.h)
SHIFT_OPS = {"mlp": 0, "attn": 1, "block": 2, "map_cls": 3, "map_mean": 4}
DISTANCES = {"l2": 0, "l1": 1, "cos": 2}


class ModelSpec:
    """Width, heads (head dim 64), MLP hidden width, LN eps, dtype, class token flag, the
    score: score_op "mlp" (the method), "attn" or "block" (shifts), "map_cls" / "map_mean"
    (attention-map baselines, Eq. (2) / (3)); score_dist "l2" (the method), "l1" or "cos";
    and attn_map: every block's attention stores its map (the non-fused comparison)."""

    def __init__(self, C: int, heads: int, hidden: int, dtype: torch.dtype = torch.bfloat16,
                 has_cls: bool = True, ln_eps: float = 1e-6, score_op: str = "mlp",
                 score_dist: str = "l2", attn_map: bool = False):
        if dtype not in _DT:
            raise TypeError(f"dtype must be float32 or bfloat16, got {dtype}")
        if score_op not in SHIFT_OPS:
            raise ValueError(f"score_op must be one of {sorted(SHIFT_OPS)}, got {score_op!r}")
        if score_dist not in DISTANCES:
            raise ValueError(f"score_dist must be one of {sorted(DISTANCES)}, got {score_dist!r}")
        self.C, self.heads, self.hidden, self.dtype = C, heads, hidden, dtype
        self.has_cls, self.ln_eps = bool(has_cls), float(ln_eps)
        self.score_op, self.score_dist, self.attn_map = score_op, score_dist, bool(attn_map)

    def desc(self) -> N.ModelDesc:
        return N.ModelDesc(self.C, self.heads, self.hidden, self.ln_eps, _DT[self.dtype],
                           int(self.has_cls), SHIFT_OPS[self.score_op],
                           DISTANCES[self.score_dist], int(self.attn_map))

    def weight_shapes(self):
        C, Hd = self.C, self.hidden
        return {"ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,),
                "w_proj": (C, C), "b_proj": (C,), "ln2_g": (C,), "ln2_b": (C,),
                "w_fc1": (Hd, C), "b_fc1": (Hd,), "w_fc2": (C, Hd), "b_fc2": (C,)}


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t.data_ptr()


def _weights(spec: ModelSpec, w: Dict[str, torch.Tensor]) -> N.BlockWeights:
    shapes = spec.weight_shapes()
    return N.BlockWeights(*[_dev(w[n], n, spec.dtype, shapes[n]) for n in BLOCK_FIELDS])


def workspace_bytes(spec: ModelSpec, depth: int, B: int, L: int) -> int:
    d = spec.desc()
    n = lib().rs_workspace_bytes(ctypes.byref(d), depth, B, L)
    if n == 0:
        raise ValueError("invalid model description for the workspace query")
    return int(n)


def _workspace(spec, depth, B, L, device):
    return torch.empty(workspace_bytes(spec, depth, B, L), dtype=torch.uint8, device=device)


def block_forward(spec: ModelSpec, w: Dict[str, torch.Tensor], x: torch.Tensor, keep_k: int,
                  want_y: bool = True, want_scores: bool = True,
                  workspace: Optional[torch.Tensor] = None):
    """One pre-LN block plus selection.  x [B, L, C].  Returns a dict with y (block
    output, or None), scores [B, L] fp32 (or None), kept_idx [B, keep_k] int32 and
    y_kept [B, keep_k, C]."""
    B, L, C = x.shape
    _dev(x, "x", spec.dtype, (B, L, spec.C))
    dev = x.device
    y = torch.empty_like(x) if want_y else None
    s = torch.empty(B, L, dtype=torch.float32, device=dev) if want_scores else None
    kept = torch.empty(B, keep_k, dtype=torch.int32, device=dev)
    yk = torch.empty(B, keep_k, C, dtype=x.dtype, device=dev)
    ws = _workspace(spec, 1, B, L, dev) if workspace is None else workspace
    d, wt = spec.desc(), _weights(spec, w)
    N.check("rs_block_forward", lib().rs_block_forward(
        ctypes.byref(d), ctypes.byref(wt), x.data_ptr(), B, L, keep_k,
        y.data_ptr() if y is not None else None, s.data_ptr() if s is not None else None,
        kept.data_ptr(), yk.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return {"y": y, "scores": s, "kept_idx": kept, "y_kept": yk}


def score(fx: torch.Tensor, x: torch.Tensor, dist: str = "l2") -> torch.Tensor:
    """D(fx, x) per row over the last axis (dist "l2": || fx - x ||_2, "l1", or "cos":
    cosine distance); fx, x [B, L, C] -> [B, L] fp32."""
    if fx.shape != x.shape or fx.dtype != x.dtype or x.dim() != 3:
        raise ValueError("fx and x must be [B, L, C] tensors of one shape and dtype")
    B, L, C = x.shape
    _dev(fx, "fx", x.dtype)
    _dev(x, "x", x.dtype)
    if x.dtype not in _DT:
        raise TypeError("dtype must be float32 or bfloat16")
    if dist not in DISTANCES:
        raise ValueError(f"dist must be one of {sorted(DISTANCES)}, got {dist!r}")
    s = torch.empty(B, L, dtype=torch.float32, device=x.device)
    if dist == "l2":
        N.check("rs_score", lib().rs_score(fx.data_ptr(), x.data_ptr(), B, L, C, _DT[x.dtype],
                                           s.data_ptr(), _stream()))
    else:
        N.check("rs_score_dist", lib().rs_score_dist(fx.data_ptr(), x.data_ptr(), B, L, C,
                                                     _DT[x.dtype], DISTANCES[dist], s.data_ptr(),
                                                     _stream()))
    return s


def attention(spec: ModelSpec, qkv: torch.Tensor, want_map: bool = False,
              want_cls: bool = False, want_mean: bool = False):
    """Multi-head attention of qkv [B, L, 3C].  Returns (out [B, L, C], map
    [B, H, L, Lpad] or None, Eq. (2) scores [B, L] or None, Eq. (3) scores [B, L] or None).
    Without any of the optional outputs the fused kernel runs (no map is formed)."""
    B, L, C3 = qkv.shape
    _dev(qkv, "qkv", spec.dtype, (B, L, 3 * spec.C))
    dev = qkv.device
    out = torch.empty(B, L, spec.C, dtype=spec.dtype, device=dev)
    lpad = (L + 7) // 8 * 8
    amap = torch.empty(B, spec.heads, L, lpad, dtype=spec.dtype, device=dev) if want_map else None
    sc = torch.empty(B, L, dtype=torch.float32, device=dev) if want_cls else None
    sm = torch.empty(B, L, dtype=torch.float32, device=dev) if want_mean else None
    d = spec.desc()
    nws = int(lib().rs_attention_workspace_bytes(ctypes.byref(d), B, L)) if (want_cls or want_mean) else 0
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
    ptr = lambda t: t.data_ptr() if t is not None else None
    N.check("rs_attention", lib().rs_attention(ctypes.byref(d), qkv.data_ptr(), B, L, out.data_ptr(),
                                               ptr(amap), ptr(sc), ptr(sm), ws.data_ptr(), nws,
                                               _stream()))
    return out, amap, sc, sm


def topk_gather(scores: torch.Tensor, x: Optional[torch.Tensor], keep_k: int, has_cls: bool):
    """Per-sample top-keep_k of scores [B, L] (fp32).  Returns (kept_idx [B, keep_k] int32,
    x_kept [B, keep_k, C] or None when x is None)."""
    B, L = scores.shape
    _dev(scores, "scores", torch.float32)
    kept = torch.empty(B, keep_k, dtype=torch.int32, device=scores.device)
    if x is not None:
        _dev(x, "x", None, (B, L, x.shape[2]))
        if x.dtype not in _DT:
            raise TypeError("dtype must be float32 or bfloat16")
        C, dt = x.shape[2], _DT[x.dtype]
        xk = torch.empty(B, keep_k, C, dtype=x.dtype, device=x.device)
        xp, xkp = x.data_ptr(), xk.data_ptr()
    else:
        C, dt, xk, xp, xkp = 0, N.RS_F32, None, None, None
    N.check("rs_topk_gather", lib().rs_topk_gather(scores.data_ptr(), xp, B, L, C, dt, keep_k,
                                                   int(has_cls), kept.data_ptr(), xkp, _stream()))
    return kept, xk


def encoder_out_len(depth: int, L: int, prune_layers: Sequence[int],
                    keep_ratios: Sequence[float]) -> int:
    out = ctypes.c_int(0)
    N.check("rs_encoder_out_len", lib().rs_encoder_out_len(
        depth, L, N.int_array(prune_layers), N.dbl_array(keep_ratios), len(prune_layers),
        ctypes.byref(out)))
    return out.value


class Encoder:
    """A whole encoder bound to fixed (B, L) with its workspace and outputs allocated
    once, so repeated forward() calls allocate nothing."""

    def __init__(self, spec: ModelSpec, blocks: List[Dict[str, torch.Tensor]], B: int, L: int,
                 prune_layers: Sequence[int], keep_ratios: Sequence[float], device="cuda"):
        self.spec, self.B, self.L = spec, B, L
        self.depth = len(blocks)
        self.prune = list(prune_layers)
        self.ratios = [float(r) for r in keep_ratios]
        self.L_final = encoder_out_len(self.depth, L, self.prune, self.ratios)
        self._blocks = blocks  # keep the tensors alive
        self._w = (N.BlockWeights * self.depth)(*[_weights(spec, w) for w in blocks])
        self._desc = spec.desc()
        self._pl, self._kr = N.int_array(self.prune), N.dbl_array(self.ratios)
        self.workspace = _workspace(spec, self.depth, B, L, device)
        self.out = torch.empty(B, self.L_final, spec.C, dtype=spec.dtype, device=device)
        self.out_idx = torch.empty(B, self.L_final, dtype=torch.int32, device=device)

    def forward(self, x: torch.Tensor):
        _dev(x, "x", self.spec.dtype, (self.B, self.L, self.spec.C))
        N.check("rs_encoder_forward", lib().rs_encoder_forward(
            ctypes.byref(self._desc), self._w, self.depth, x.data_ptr(), self.B, self.L,
            self._pl, self._kr, len(self.prune), self.out.data_ptr(), self.out_idx.data_ptr(),
            self.workspace.data_ptr(), self.workspace.numel(), _stream()))
        return self.out, self.out_idx


def encoder_forward(spec: ModelSpec, blocks: List[Dict[str, torch.Tensor]], x: torch.Tensor,
                    prune_layers: Sequence[int], keep_ratios: Sequence[float]):
    """Whole encoder with progressive pruning.  Returns (out [B, L_final, C],
    out_idx [B, L_final] original token ids)."""
    B, L, _ = x.shape
    enc = Encoder(spec, blocks, B, L, prune_layers, keep_ratios, device=x.device)
    out, idx = enc.forward(x)
    return out, idx


class ImageSpec:
    """Pixel input geometry: frames (1 for an image), channels, height, width, patch size
    P (8, 16 or 32).  Tokens per sample: has_cls + frames * (height/P) * (width/P)."""

    def __init__(self, frames: int = 1, in_chans: int = 3, height: int = 224, width: int = 224,
                 patch: int = 16):
        self.frames, self.in_chans, self.height, self.width, self.patch = (
            int(frames), int(in_chans), int(height), int(width), int(patch))

    def desc(self) -> N.ImageDesc:
        return N.ImageDesc(self.frames, self.in_chans, self.height, self.width, self.patch)

    def tokens(self, has_cls: bool) -> int:
        P = self.patch
        return int(has_cls) + self.frames * (self.height // P) * (self.width // P)

    def image_shape(self, B: int):
        return (B, self.frames, self.in_chans, self.height, self.width)


def _embed(spec: ModelSpec, img: ImageSpec, e: Dict[str, torch.Tensor]) -> N.EmbedWeights:
    C, L = spec.C, img.tokens(spec.has_cls)
    shapes = {"w_patch": (C, img.in_chans * img.patch ** 2), "b_patch": (C,), "cls": (C,),
              "pos": (L, C)}
    ptrs = []
    for n in N.EMBED_FIELDS:
        if n == "cls" and not spec.has_cls:
            ptrs.append(None)
        else:
            ptrs.append(_dev(e[n], n, spec.dtype, shapes[n]))
    return N.EmbedWeights(*ptrs)


def _head(spec: ModelSpec, h: Dict[str, torch.Tensor], pool: str) -> N.HeadWeights:
    if pool not in ("cls", "mean"):
        raise ValueError(f"pool must be 'cls' or 'mean', got {pool!r}")
    n_out = h["w_head"].shape[0]
    shapes = {"ln_g": (spec.C,), "ln_b": (spec.C,), "w_head": (n_out, spec.C), "b_head": (n_out,)}
    ptrs = [_dev(h[n], n, spec.dtype, shapes[n]) for n in N.HEAD_FIELDS]
    return N.HeadWeights(*ptrs, n_out, N.RS_POOL_CLS if pool == "cls" else N.RS_POOL_MEAN)


def patch_embed(spec: ModelSpec, img: ImageSpec, emb: Dict[str, torch.Tensor],
                images: torch.Tensor) -> torch.Tensor:
    """Patch embedding: images [B, frames, in_chans, H, W] -> tokens [B, L, C]."""
    B = images.shape[0]
    _dev(images, "images", spec.dtype, img.image_shape(B))
    tokens = torch.empty(B, img.tokens(spec.has_cls), spec.C, dtype=spec.dtype, device=images.device)
    d, idesc, e = spec.desc(), img.desc(), _embed(spec, img, emb)
    N.check("rs_patch_embed", lib().rs_patch_embed(ctypes.byref(d), ctypes.byref(idesc),
                                                   ctypes.byref(e), images.data_ptr(), B,
                                                   tokens.data_ptr(), _stream()))
    return tokens


def head(spec: ModelSpec, hw: Dict[str, torch.Tensor], x: torch.Tensor, pool: str):
    """Final LayerNorm, pooling ('cls' or 'mean') and head of x [B, L, C].  Returns
    (features [B, C], logits [B, n_out])."""
    B, L, C = x.shape
    _dev(x, "x", spec.dtype, (B, L, spec.C))
    h = _head(spec, hw, pool)
    feat = torch.empty(B, spec.C, dtype=spec.dtype, device=x.device)
    logits = torch.empty(B, h.n_out, dtype=spec.dtype, device=x.device)
    ws = torch.empty(int(lib().rs_head_workspace_bytes(B, L, spec.C)), dtype=torch.uint8,
                     device=x.device)
    d = spec.desc()
    N.check("rs_head", lib().rs_head(ctypes.byref(d), ctypes.byref(h), x.data_ptr(), B, L,
                                     feat.data_ptr(), logits.data_ptr(), ws.data_ptr(), ws.numel(),
                                     _stream()))
    return feat, logits


class ViT:
    """The whole forward pass (patch embedding, pruned encoder, head) bound to a batch
    size, with its workspace and outputs allocated once."""

    def __init__(self, spec: ModelSpec, img: ImageSpec, emb: Dict[str, torch.Tensor],
                 blocks: List[Dict[str, torch.Tensor]], hw: Dict[str, torch.Tensor], pool: str,
                 B: int, prune_layers: Sequence[int], keep_ratios: Sequence[float],
                 device="cuda"):
        self.spec, self.img, self.B = spec, img, B
        self.depth = len(blocks)
        self.L = img.tokens(spec.has_cls)
        self.prune = list(prune_layers)
        self.ratios = [float(r) for r in keep_ratios]
        self.L_final = encoder_out_len(self.depth, self.L, self.prune, self.ratios)
        self._keep = (emb, blocks, hw)  # keep the tensors alive
        self._desc, self._idesc = spec.desc(), img.desc()
        self._emb = _embed(spec, img, emb)
        self._w = (N.BlockWeights * self.depth)(*[_weights(spec, w) for w in blocks])
        self._head = _head(spec, hw, pool)
        self._pl, self._kr = N.int_array(self.prune), N.dbl_array(self.ratios)
        n = lib().rs_vit_workspace_bytes(ctypes.byref(self._desc), ctypes.byref(self._idesc),
                                         self.depth, B)
        if n == 0:
            raise ValueError("invalid model or image description for the workspace query")
        self.workspace = torch.empty(int(n), dtype=torch.uint8, device=device)
        self.features = torch.empty(B, spec.C, dtype=spec.dtype, device=device)
        self.logits = torch.empty(B, self._head.n_out, dtype=spec.dtype, device=device)
        self.out_idx = torch.empty(B, self.L_final, dtype=torch.int32, device=device)

    def forward(self, images: torch.Tensor):
        _dev(images, "images", self.spec.dtype, self.img.image_shape(self.B))
        N.check("rs_vit_forward", lib().rs_vit_forward(
            ctypes.byref(self._desc), ctypes.byref(self._idesc), ctypes.byref(self._emb), self._w,
            self.depth, ctypes.byref(self._head), images.data_ptr(), self.B, self._pl, self._kr,
            len(self.prune), self.features.data_ptr(), self.logits.data_ptr(),
            self.out_idx.data_ptr(), self.workspace.data_ptr(), self.workspace.numel(),
            _stream()))
        return self.features, self.logits, self.out_idx


def vit_forward(spec: ModelSpec, img: ImageSpec, emb, blocks, hw, pool: str,
                images: torch.Tensor, prune_layers: Sequence[int], keep_ratios: Sequence[float]):
    """Whole forward pass.  Returns (features [B, C], logits [B, n_out], out_idx
    [B, L_final])."""
    m = ViT(spec, img, emb, blocks, hw, pool, images.shape[0], prune_layers, keep_ratios,
            device=images.device)
    return m.forward(images)


def set_max_lanes(lanes: int) -> None:
    """Most concurrent lanes (streams) the encoder may split a batch into: 1 .. 4
    (default 2)."""
    N.check("rs_set_max_lanes", lib().rs_set_max_lanes(int(lanes)))


def get_max_lanes() -> int:
    """The current most-lanes setting of the encoder (see set_max_lanes)."""
    return int(lib().rs_get_max_lanes())


class KernelTimer:
    """HIP-event timing of one kernel class inside the library (see rs_timing_begin)."""

    def __init__(self, kernel: str):
        self.kid = KERNELS.index(kernel)

    def __enter__(self):
        N.check("rs_timing_begin", lib().rs_timing_begin(self.kid))
        return self

    def __exit__(self, *exc):
        ms, n, work = ctypes.c_float(), ctypes.c_int(), ctypes.c_double()
        st = lib().rs_timing_end(ctypes.byref(ms), ctypes.byref(n), ctypes.byref(work))
        if exc[0] is None:
            N.check("rs_timing_end", st)
        self.total_ms, self.launches, self.work = ms.value, n.value, work.value
        return False

"""Seeded synthetic inputs for the Representation Shift hot path.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds *no* arithmetic of the method: only workload shapes (as data), seeded random
draws and the bf16 storage rounding of those draws.  Everything the method computes
lives twice, independently: in ``oracle/`` (fp64 CPU) and in the HIP library.

Workloads stand in for the pages' datasets (ImageNet-1K for DeiT, the video-text
sets for UMT; "Representation Shift: Unifying Token Compression with
FlashAttention", arXiv HTML, Sec. 4.1 and Sec. 4.2), which are not available:
token counts follow the ViT tokenisation of Sec. 3.1 (224x224 images, 16x16
patches -> 196 patches, plus a class token for DeiT; 196 patches per frame and no
class token for the video encoder).

Recipe (identical for every workload unless stated):
  * generator: ``numpy.random.default_rng([seed, block, tensor_id])``;
  * block input x ~ N(0, 1);
  * Linear weights ~ N(0, 0.02^2), stored [out][in];
  * ``init="paper"``: Linear biases 0, LayerNorm gamma = 1, beta = 0;
    ``init="full"`` (parity tests only, so that every bias and affine term is
    exercised): biases ~ N(0, 0.02^2), gamma ~ 1 + N(0, 0.1^2), beta ~ N(0, 0.1^2);
  * ``spread=True`` multiplies each token row of x by a_i ~ U(0.5, 1.5), which
    widens the score distribution so that near-ties become rare;
  * ``offset`` / ``spikes`` (parity tests of the folded LayerNorm): rows with a large
    common offset and a few channels of magnitude ~50, so that |mean| / std of a row is
    large, the regime in which LayerNorm statistics cancel;
  * bf16 workloads: values are drawn in fp32 and rounded to bf16 (round to
    nearest, ties to even) here, so the GPU path and the oracle see the very same
    numbers; arrays are returned as float32 holding bf16-representable values;
  * whole forward pass: pixels ~ N(0, 1) (images after per-channel normalisation),
    patch weights ~ N(0, 0.02^2), class token and position table ~ N(0, 0.02^2),
    head weights ~ N(0, 0.02^2), final LayerNorm as the blocks' (``init``);
    geometry 224 x 224 pixels, 16 x 16 patches, 3 channels, frames = the workload's
    patch tokens / 196; 1000 classes and class-token pooling for image workloads,
    a 512-wide head and mean pooling for video workloads.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

# tensor ids inside one block's weight set (also the order of the C struct fields)
WEIGHT_NAMES = (
    "ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
    "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2",
)
_INPUT_BLOCK_TAG = 1_000_000
_SPREAD_TAG = 1_000_001
_IMAGE_TAG = 1_000_002
_EMBED_TAG = 1_000_003
_HEAD_TAG = 1_000_004
_SPIKE_TAG = 1_000_005


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and pruning schedule of one synthetic workload (data only)."""
    name: str
    B: int                 # samples (images or clips)
    L: int                 # tokens per sample at the encoder input
    C: int                 # width
    heads: int             # attention heads, head dim = C / heads = 64
    hidden: int            # MLP hidden width
    depth: int             # encoder blocks
    dtype: str             # "f32" or "bf16"
    has_cls: bool          # class token at index 0 (DeiT) or none (video)
    prune_layers: tuple    # 0-based block indices after whose MLP tokens are pruned
    keep_ratios: tuple     # fraction of the current tokens kept at each prune block
    unit: str              # throughput unit of one sample
    ln_eps: float = 1e-6

    @property
    def head_dim(self) -> int:
        return self.C // self.heads


WORKLOADS: Dict[str, Workload] = {
    # one DeiT-T block in fp32: batch 2, 197 tokens, keep 138 (70%, class token kept)
    "deit_t_block": Workload("deit_t_block", 2, 197, 192, 3, 768, 1, "f32", True,
                             (0,), (0.7,), "blocks"),
    # DeiT-S-shaped 12-block encoder, bf16, pruning after blocks 3/6/9 keeping 70%
    "deit_s": Workload("deit_s", 256, 197, 384, 6, 1536, 12, "bf16", True,
                       (3, 6, 9), (0.7, 0.7, 0.7), "img"),
    # DeiT-B-shaped, bf16, pruning after blocks 2/5/8 keeping 65%
    "deit_b": Workload("deit_b", 128, 197, 768, 12, 3072, 12, "bf16", True,
                       (2, 5, 8), (0.65, 0.65, 0.65), "img"),
    # UMT-B-shaped video encoder: 8 clips x (8 frames x 196 patches), no class token
    "umt_b": Workload("umt_b", 8, 1568, 768, 12, 3072, 12, "bf16", False,
                      (1, 4, 7), (0.5, 0.5, 0.5), "vid"),
    # UMT-L-shaped video encoder: 4 clips x 1568 tokens, 24 blocks
    "umt_l": Workload("umt_l", 4, 1568, 1024, 16, 4096, 24, "bf16", False,
                      (2, 6, 10, 14), (0.5, 0.5, 0.5, 0.5), "vid"),
    # The pages' own settings.  DeiT-T/S/B on ImageNet-1K (Sec. 4.2, Table 5): 20 % of the
    # current tokens dropped after the blocks the pages number 1, 4, 7 (0-based 0, 3, 6);
    # batch 512 for throughput.
    "deit_t512": Workload("deit_t512", 512, 197, 192, 3, 768, 12, "bf16", True,
                          (0, 3, 6), (0.8, 0.8, 0.8), "img"),
    "deit_s512": Workload("deit_s512", 512, 197, 384, 6, 1536, 12, "bf16", True,
                          (0, 3, 6), (0.8, 0.8, 0.8), "img"),
    "deit_b512": Workload("deit_b512", 512, 197, 768, 12, 3072, 12, "bf16", True,
                          (0, 3, 6), (0.8, 0.8, 0.8), "img"),
    # UMT-B/L at 12 frames x 196 patches = 2352 tokens, no class token, batch 20 (Sec. 4.1
    # throughput setting); 20 % (retrieval, Table 2) or 10 % (QA, Table 4) of the current
    # tokens dropped after each of the first three blocks.
    "umt_b12f_ret": Workload("umt_b12f_ret", 20, 2352, 768, 12, 3072, 12, "bf16", False,
                             (0, 1, 2), (0.8, 0.8, 0.8), "vid"),
    "umt_b12f_qa": Workload("umt_b12f_qa", 20, 2352, 768, 12, 3072, 12, "bf16", False,
                            (0, 1, 2), (0.9, 0.9, 0.9), "vid"),
    "umt_l12f_ret": Workload("umt_l12f_ret", 20, 2352, 1024, 16, 4096, 24, "bf16", False,
                             (0, 1, 2), (0.8, 0.8, 0.8), "vid"),
    "umt_l12f_qa": Workload("umt_l12f_qa", 20, 2352, 1024, 16, 4096, 24, "bf16", False,
                            (0, 1, 2), (0.9, 0.9, 0.9), "vid"),
}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32.

    Finite inputs only (the generators never produce NaN or Inf)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


def _finish(a: np.ndarray, dtype: str) -> np.ndarray:
    a = a.astype(np.float32, copy=False)
    return round_to_bf16(a) if dtype == "bf16" else np.ascontiguousarray(a)


def make_input(wl: Workload, seed: int = 0, B: Optional[int] = None, L: Optional[int] = None,
               spread: bool = False, offset: float = 0.0, spikes: int = 0,
               spike: float = 50.0) -> np.ndarray:
    """Block/encoder input x of shape [B, L, C], x ~ N(0, 1).

    ``offset`` adds a constant to every element (rows far from zero mean, as residual
    streams with a large common component are); ``spikes`` picks that many channels
    (seeded, the same for every token) and adds +-``spike`` to them, signs alternating
    (a few large-magnitude channels)."""
    B = wl.B if B is None else B
    L = wl.L if L is None else L
    rng = np.random.default_rng([seed, _INPUT_BLOCK_TAG, 0])
    x = rng.standard_normal((B, L, wl.C), dtype=np.float32)
    if spread:
        a = np.random.default_rng([seed, _SPREAD_TAG, 0]).uniform(0.5, 1.5, size=(B, L, 1))
        x = x * a.astype(np.float32)
    if offset:
        x = x + np.float32(offset)
    if spikes:
        ch = np.random.default_rng([seed, _SPIKE_TAG, 0]).choice(wl.C, size=spikes, replace=False)
        sign = np.where(np.arange(spikes) % 2 == 0, 1.0, -1.0).astype(np.float32)
        x[..., ch] += np.float32(spike) * sign
    return _finish(x, wl.dtype)


def make_block_weights(wl: Workload, block: int, seed: int = 0, init: str = "paper",
                       zero: tuple = ()) -> Dict[str, np.ndarray]:
    """Weights of one pre-LN block; every Linear is stored [out][in].

    ``zero`` names tensors to be set to exactly 0 (closed-form tests)."""
    if init not in ("paper", "full"):
        raise ValueError(init)
    C, Hd = wl.C, wl.hidden
    shapes = {
        "ln1_g": (C,), "ln1_b": (C,), "w_qkv": (3 * C, C), "b_qkv": (3 * C,),
        "w_proj": (C, C), "b_proj": (C,), "ln2_g": (C,), "ln2_b": (C,),
        "w_fc1": (Hd, C), "b_fc1": (Hd,), "w_fc2": (C, Hd), "b_fc2": (C,),
    }
    out = {}
    for tid, name in enumerate(WEIGHT_NAMES):
        rng = np.random.default_rng([seed, block, tid])
        shp = shapes[name]
        if name.startswith("w_"):
            a = rng.standard_normal(shp, dtype=np.float32) * np.float32(0.02)
        elif name.endswith("_g"):
            a = (np.ones(shp, np.float32) if init == "paper"
                 else 1.0 + 0.1 * rng.standard_normal(shp, dtype=np.float32))
        elif name.endswith("_b") and name.startswith("ln"):
            a = (np.zeros(shp, np.float32) if init == "paper"
                 else 0.1 * rng.standard_normal(shp, dtype=np.float32))
        else:  # Linear bias
            a = (np.zeros(shp, np.float32) if init == "paper"
                 else 0.02 * rng.standard_normal(shp, dtype=np.float32))
        if name in zero:
            a = np.zeros(shp, np.float32)
        out[name] = _finish(a, wl.dtype)
    return out


@dataclasses.dataclass(frozen=True)
class Geometry:
    """Pixel input and head of a whole forward pass (data only)."""
    frames: int
    in_chans: int
    height: int
    width: int
    patch: int
    n_out: int
    pool: str              # "cls" or "mean"

    def tokens(self, has_cls: bool) -> int:
        return int(has_cls) + self.frames * (self.height // self.patch) * (self.width // self.patch)


def geometry(wl: Workload) -> Geometry:
    """224 x 224 images cut into 16 x 16 patches (196 per frame); the frame count follows
    from the workload's token count."""
    patches = wl.L - int(wl.has_cls)
    if patches % 196:
        raise ValueError(f"{wl.name}: {patches} patch tokens is not a whole number of frames")
    return Geometry(patches // 196, 3, 224, 224, 16, 1000 if wl.has_cls else 512,
                    "cls" if wl.has_cls else "mean")


def make_images(wl: Workload, geom: Geometry, seed: int = 0, B: Optional[int] = None) -> np.ndarray:
    """Pixels [B][frames][in_chans][H][W] ~ N(0, 1)."""
    B = wl.B if B is None else B
    rng = np.random.default_rng([seed, _IMAGE_TAG, 0])
    shape = (B, geom.frames, geom.in_chans, geom.height, geom.width)
    return _finish(rng.standard_normal(shape, dtype=np.float32), wl.dtype)


def make_embed_weights(wl: Workload, geom: Geometry, seed: int = 0) -> Dict[str, np.ndarray]:
    """w_patch [C][in_chans*P*P], b_patch [C], cls [C], pos [L][C]."""
    C, L = wl.C, geom.tokens(wl.has_cls)
    shapes = {"w_patch": (C, geom.in_chans * geom.patch ** 2), "b_patch": (C,), "cls": (C,),
              "pos": (L, C)}
    out = {}
    for tid, (name, shp) in enumerate(shapes.items()):
        rng = np.random.default_rng([seed, _EMBED_TAG, tid])
        out[name] = _finish(rng.standard_normal(shp, dtype=np.float32) * np.float32(0.02), wl.dtype)
    return out


def make_head_weights(wl: Workload, geom: Geometry, seed: int = 0, init: str = "paper") -> Dict[str, np.ndarray]:
    """ln_g, ln_b [C], w_head [n_out][C], b_head [n_out]."""
    if init not in ("paper", "full"):
        raise ValueError(init)
    C, n = wl.C, geom.n_out
    out = {}
    for tid, (name, shp) in enumerate((("ln_g", (C,)), ("ln_b", (C,)), ("w_head", (n, C)),
                                       ("b_head", (n,)))):
        rng = np.random.default_rng([seed, _HEAD_TAG, tid])
        if name == "w_head":
            a = rng.standard_normal(shp, dtype=np.float32) * np.float32(0.02)
        elif name == "ln_g":
            a = (np.ones(shp, np.float32) if init == "paper"
                 else 1.0 + 0.1 * rng.standard_normal(shp, dtype=np.float32))
        elif name == "ln_b":
            a = (np.zeros(shp, np.float32) if init == "paper"
                 else 0.1 * rng.standard_normal(shp, dtype=np.float32))
        else:
            a = (np.zeros(shp, np.float32) if init == "paper"
                 else 0.02 * rng.standard_normal(shp, dtype=np.float32))
        out[name] = _finish(a, wl.dtype)
    return out


def make_encoder_weights(wl: Workload, seed: int = 0, init: str = "paper",
                         depth: Optional[int] = None) -> List[Dict[str, np.ndarray]]:
    depth = wl.depth if depth is None else depth
    return [make_block_weights(wl, b, seed, init) for b in range(depth)]


def make_scores(B: int, L: int, seed: int = 0, kind: str = "normal") -> np.ndarray:
    """Synthetic per-token scores [B, L] float32 for selection-only tests.

    kind="normal": |N(0,1)| * 10 + 20 (positive, like L2 norms);
    kind="ties":   small integers 0..7, so many exact ties;
    kind="signed": N(0, 1) with both signs."""
    rng = np.random.default_rng([seed, _INPUT_BLOCK_TAG, 7])
    if kind == "normal":
        s = np.abs(rng.standard_normal((B, L))) * 10 + 20
    elif kind == "ties":
        s = rng.integers(0, 8, size=(B, L)).astype(np.float64)
    elif kind == "signed":
        s = rng.standard_normal((B, L))
    else:
        raise ValueError(kind)
    return s.astype(np.float32)

"""ctypes binding of librs.so (include/rs.h).  Argument marshalling only: every step
of the hot path runs in the library's HIP kernels; torch supplies device memory and
the current stream.  If the library is missing, every call raises."""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librs.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "rs.h")

RS_OK, RS_ERR_INVALID_ARG, RS_ERR_UNSUPPORTED, RS_ERR_WORKSPACE, RS_ERR_HIP = range(5)
RS_F32, RS_BF16 = 0, 1
KERNELS = ("ln_prep", "qkv", "attention", "proj", "fc1", "fc2_score", "topk", "gather", "score",
           "patch_embed", "head", "map_score", "mlp")
RS_POOL_CLS, RS_POOL_MEAN = 0, 1

# field order of rs_embed_weights and of the pointer fields of rs_head_weights
EMBED_FIELDS = ("w_patch", "b_patch", "cls", "pos")
HEAD_FIELDS = ("ln_g", "ln_b", "w_head", "b_head")
# field order of rs_block_weights
BLOCK_FIELDS = ("ln1_g", "ln1_b", "w_qkv", "b_qkv", "w_proj", "b_proj",
                "ln2_g", "ln2_b", "w_fc1", "b_fc1", "w_fc2", "b_fc2")

c_int, c_size_t, c_void_p, c_float, c_double = (ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p,
                                                 ctypes.c_float, ctypes.c_double)
P_INT = ctypes.POINTER(c_int)
P_DBL = ctypes.POINTER(c_double)


class ModelDesc(ctypes.Structure):
    _fields_ = [("C", c_int), ("heads", c_int), ("hidden", c_int), ("ln_eps", c_float),
                ("dtype", c_int), ("has_cls", c_int), ("score_op", c_int),
                ("score_dist", c_int), ("attn_map", c_int)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in BLOCK_FIELDS]


class ImageDesc(ctypes.Structure):
    _fields_ = [("frames", c_int), ("in_chans", c_int), ("height", c_int), ("width", c_int),
                ("patch", c_int)]


class EmbedWeights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in EMBED_FIELDS]


class HeadWeights(ctypes.Structure):
    _fields_ = [("ln_g", c_void_p), ("ln_b", c_void_p), ("w_head", c_void_p),
                ("b_head", c_void_p), ("n_out", c_int), ("pool", c_int)]


class RSError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed (status {status}): {msg}")
        self.status = status


_lib = None


def lib():
    """Load librs.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m vit_token_pruning_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    P_DESC, P_W = ctypes.POINTER(ModelDesc), ctypes.POINTER(BlockWeights)
    P_IMG, P_EMB = ctypes.POINTER(ImageDesc), ctypes.POINTER(EmbedWeights)
    P_HEAD = ctypes.POINTER(HeadWeights)
    sig = {
        "rs_block_forward": (c_int, [P_DESC, P_W, c_void_p, c_int, c_int, c_int, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "rs_score": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
        "rs_score_dist": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_void_p,
                                  c_void_p]),
        "rs_topk_gather": (c_int, [c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int,
                                   c_void_p, c_void_p, c_void_p]),
        "rs_encoder_forward": (c_int, [P_DESC, P_W, c_int, c_void_p, c_int, c_int, P_INT, P_DBL,
                                       c_int, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
        "rs_encoder_out_len": (c_int, [c_int, c_int, P_INT, P_DBL, c_int, P_INT]),
        "rs_attention": (c_int, [P_DESC, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_size_t, c_void_p]),
        "rs_attention_workspace_bytes": (c_size_t, [P_DESC, c_int, c_int]),
        "rs_attention_noalloc": (c_int, [P_DESC, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p]),
        "rs_patch_embed": (c_int, [P_DESC, P_IMG, P_EMB, c_void_p, c_int, c_void_p, c_void_p]),
        "rs_head": (c_int, [P_DESC, P_HEAD, c_void_p, c_int, c_int, c_void_p, c_void_p, c_void_p,
                            c_size_t, c_void_p]),
        "rs_head_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
        "rs_vit_forward": (c_int, [P_DESC, P_IMG, P_EMB, P_W, c_int, P_HEAD, c_void_p, c_int, P_INT,
                                   P_DBL, c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
        "rs_vit_workspace_bytes": (c_size_t, [P_DESC, P_IMG, c_int, c_int]),
        "rs_workspace_bytes": (c_size_t, [P_DESC, c_int, c_int, c_int]),
        "rs_last_error": (ctypes.c_char_p, []),
        "rs_set_max_lanes": (c_int, [c_int]),
        "rs_get_max_lanes": (c_int, []),
        "rs_probe_throughput": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p]),
        "rs_timing_begin": (c_int, [c_int]),
        "rs_timing_end": (c_int, [ctypes.POINTER(c_float), P_INT, P_DBL]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def declared_symbols():
    """Names of the functions include/rs.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rs_[a-z_]+)\s*\(", text)))


def check(fn, status):
    if status != RS_OK:
        raise RSError(fn, status, lib().rs_last_error().decode())


def int_array(vals):
    vals = list(vals)
    return (c_int * max(1, len(vals)))(*vals)


def dbl_array(vals):
    vals = list(vals)
    return (c_double * max(1, len(vals)))(*vals)

"""Representation Shift — fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this module.  The product (the HIP library
and its Python binding) never imports, calls or links anything here, and this
module imports nothing from the product.

It is a plain, slow, obviously correct restatement of what the method computes,
written from "Representation Shift: Unifying Token Compression with
FlashAttention" (arXiv HTML page), in float64 NumPy:

  * Sec. 3.1, Eq. (1): self-attention Softmax(Q K^T / sqrt(.)) V with [Q, K, V] = x W;
    pruning leaves a reduced set of N - r tokens.
  * Sec. 3.3, Eq. (5) and Eq. (6): the pre-LN block
        x'   = SA(LN(x)) + x
        x_hat = MLP(LN(x')) + x'
  * Sec. 3.2, Eq. (4) with Sec. 3.3 case (ii) and the L2 distance: the score of a
    token is || MLP(LN(x')) - x' ||_2.
  * Sec. 3.2 (toy experiments) and Sec. 4.1 / 4.2: the tokens with the lowest
    scores are dropped, the same count for every sample, progressively over the
    listed layers.
  * Sec. 3.3, "Operation choice" and "Distance metrics": the ablation variants of the
    score -- through the attention sublayer D(SA(LN(x)), x), the MLP sublayer
    D(MLP(LN(x')), x') (the method) or the whole block D(x_hat, x); with the L2 norm
    (the method), the L1 norm, or the cosine distance 1 - a.b / (|a| |b|).
  * Sec. 3.1: an H x W image is cut into N = (H/P)(W/P) patches of P x P pixels, the
    tokens the encoder runs on; the model ends in a final LayerNorm and a linear head
    (the DeiT and UMT models the pages run unchanged).
  * Sec. 3.1, Eq. (2) and Eq. (3): the attention-map importance scores the pages compare
    against (comparison baselines, not the method): the class token's attention row, or
    the mean over all queries of the attention rows.

Readings taken where the pages leave a step open (each also listed in the design
notes of the repository):
  * multi-head attention: the scale is 1/sqrt(head_dim) per head (Eq. (1) is
    written single-head, where head_dim = C); heads are consecutive 64-column
    groups of Q, K and V; the attention output goes through an output projection
    with bias (standard in the DeiT/UMT models the pages run unchanged);
  * MLP = fc1 (C -> hidden) + GELU (erf form) + fc2 (hidden -> C), both with bias;
  * LayerNorm: biased variance, eps a parameter (1e-6 in every workload);
  * the score subtracts x' from MLP(LN(x')) literally (not x_hat - x');
  * SA(LN(x)) in the attention variant is the attention sublayer's output, i.e. after
    the output projection and its bias (the term Eq. (5) adds to x);
  * cosine distance: 1 - a.b / max(|a| |b|, 1e-8), so a zero vector is at distance 1
    (the pages give no rule for zero norms);
  * selection: order by score descending, ties to the lower token index, NaN
    lowest, the class token (index 0) always kept when present; kept tokens are
    emitted in ascending original order;
  * schedule: pruning at block b uses block b's MLP score and compacts block b's
    output; the kept count is floor(r * L + 1/2) of the current L (counting the
    class token), evaluated in IEEE double;
  * patch embedding: a P x P, stride-P convolution with bias, i.e. each patch
    flattened channel-major (channel, row, column) times a [C][Cin*P*P] weight; tokens
    in raster order of the patch grid, frame by frame for video (frame-major); a
    learned class token first when present; a learned position table [L][C] added to
    every token (class token included);
  * head: the final LayerNorm of every token, then the class token's normalised row
    (image models with a class token) or the mean of all tokens' normalised rows
    (video models), then a Linear with bias;
  * attention-map scores with several heads: Eq. (2) / Eq. (3) per head (each head's own
    map, scaled by 1/sqrt(head_dim) as in the attention itself), averaged over the heads;
    the map is the one the block's attention forms (after LN1); all N queries count in
    Eq. (3), the class token's included.

Parity status: every function here is pinned by the tests in
``tests/test_oracle_pins.py`` (closed forms, textbook identities, brute force on
tiny inputs, and the GFLOPs the pages print); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64


# ----------------------------------------------------------------------------- pieces

def layer_norm(z: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float) -> np.ndarray:
    """LN over the last axis: (z - mean) / sqrt(var + eps) * gamma + beta, biased var.

    The LN of Eq. (5)/(6); the pages do not spell it out, this is the standard one."""
    z = np.asarray(z, F64)
    mu = z.mean(axis=-1, keepdims=True)
    var = ((z - mu) ** 2).mean(axis=-1, keepdims=True)
    return (z - mu) / np.sqrt(var + eps) * np.asarray(gamma, F64) + np.asarray(beta, F64)


def linear(z: np.ndarray, w: np.ndarray, b: np.ndarray) -> np.ndarray:
    """z W^T + b with W stored [out][in] (so that [Q,K,V] = x W of Eq. (1) has W = w^T)."""
    return np.asarray(z, F64) @ np.asarray(w, F64).T + np.asarray(b, F64)


def gelu(z: np.ndarray) -> np.ndarray:
    """GELU in its exact form z * Phi(z) = z/2 * (1 + erf(z / sqrt 2))."""
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax, max-subtracted (the value is the same as the plain definition)."""
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_materialised(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> np.ndarray:
    """One head of Eq. (1): forms the whole map A = Softmax(q k^T / sqrt(d)), returns A v.

    q, k, v: [L, d]."""
    q, k, v = (np.asarray(t, F64) for t in (q, k, v))
    d = q.shape[-1]
    a = softmax_rows(q @ k.T / math.sqrt(d))
    return a @ v


def attention_online(q: np.ndarray, k: np.ndarray, v: np.ndarray, block: int = 32) -> np.ndarray:
    """The same head computed key-block by key-block with a running max and sum, never
    holding more than one [L, block] slice of scores (the fused form the pages rely on,
    FlashAttention, written from the softmax algebra: rescale the partial numerator and
    denominator by exp(m_old - m_new) whenever the running maximum grows)."""
    q, k, v = (np.asarray(t, F64) for t in (q, k, v))
    L, d = q.shape
    m = np.full((L, 1), -np.inf)
    den = np.zeros((L, 1))
    num = np.zeros((L, v.shape[1]))
    for j0 in range(0, k.shape[0], block):
        s = q @ k[j0:j0 + block].T / math.sqrt(d)
        m_new = np.maximum(m, s.max(axis=1, keepdims=True))
        scale = np.exp(m - m_new)
        p = np.exp(s - m_new)
        den = den * scale + p.sum(axis=1, keepdims=True)
        num = num * scale + p @ v[j0:j0 + block]
        m = m_new
    return num / den


def attention_maps(xn: np.ndarray, w_qkv, b_qkv, heads: int) -> np.ndarray:
    """The attention maps A_h = Softmax(q_h k_h^T / sqrt(d)) of every head, [heads, L, L]
    (query rows, key columns), heads as in multi_head_attention."""
    L, C = xn.shape
    d = C // heads
    qkv = linear(xn, w_qkv, b_qkv)
    maps = []
    for h in range(heads):
        q = qkv[:, h * d:(h + 1) * d]
        k = qkv[:, C + h * d:C + (h + 1) * d]
        maps.append(softmax_rows(q @ k.T / math.sqrt(d)))
    return np.stack(maps)


def attention_map_score(maps: np.ndarray, kind: str) -> np.ndarray:
    """Token importance from attention maps [heads, L, L] (Sec. 3.1): "cls", Eq. (2), the
    class token's (query 0's) attention row; "mean", Eq. (3), the mean over the N query
    rows.  Averaged over heads.  Returns [L]."""
    maps = np.asarray(maps, F64)
    if kind == "cls":
        per_head = maps[:, 0, :]
    elif kind == "mean":
        per_head = maps.sum(axis=1) / maps.shape[1]
    else:
        raise ValueError(kind)
    return per_head.mean(axis=0)


def multi_head_attention(xn: np.ndarray, w_qkv, b_qkv, heads: int, fused: bool = False) -> np.ndarray:
    """Q|K|V = xn W_qkv^T + b (column blocks of C), split each into `heads` groups of
    d = C/heads consecutive columns, attend per head, concatenate heads. Returns [L, C]."""
    L, C = xn.shape
    d = C // heads
    qkv = linear(xn, w_qkv, b_qkv)
    q, k, v = qkv[:, :C], qkv[:, C:2 * C], qkv[:, 2 * C:]
    att = attention_online if fused else attention_materialised
    out = np.empty((L, C))
    for h in range(heads):
        sl = slice(h * d, (h + 1) * d)
        out[:, sl] = att(q[:, sl], k[:, sl], v[:, sl])
    return out


# ----------------------------------------------------------------------------- block

SHIFT_OPS = ("mlp", "attn", "block")
DISTANCES = ("l2", "l1", "cos")
MAP_SCORES = ("map_cls", "map_mean")   # Eq. (2) and Eq. (3): comparison baselines


def block_forward(x: np.ndarray, w: Dict[str, np.ndarray], heads: int, eps: float = 1e-6,
                  fused_attention: bool = False, op: str = "mlp",
                  dist: str = "l2") -> Dict[str, np.ndarray]:
    """One pre-LN block on one sample x [L, C], Eqs. (5) and (6), plus the representation
    shift (Eq. (4)) of the chosen operation and distance (Sec. 3.3; the method: MLP, L2),
    or with op "map_cls" / "map_mean" the attention-map score of Eq. (2) / Eq. (3) from
    this block's attention (dist ignored).

    Returns x_prime (Eq. 5), sa (= SA(LN(x))), mlp (= MLP(LN(x'))), x_hat (Eq. 6) and
    score [L]."""
    x = np.asarray(x, F64)
    xn1 = layer_norm(x, w["ln1_g"], w["ln1_b"], eps)
    sa = linear(multi_head_attention(xn1, w["w_qkv"], w["b_qkv"], heads, fused_attention),
                w["w_proj"], w["b_proj"])
    x_prime = sa + x                                                    # Eq. (5)
    xn2 = layer_norm(x_prime, w["ln2_g"], w["ln2_b"], eps)
    mlp = linear(gelu(linear(xn2, w["w_fc1"], w["b_fc1"])), w["w_fc2"], w["b_fc2"])
    x_hat = mlp + x_prime                                               # Eq. (6)
    if op in MAP_SCORES:
        score = attention_map_score(attention_maps(xn1, w["w_qkv"], w["b_qkv"], heads),
                                    op[4:])                             # Eq. (2) / (3)
    else:
        # Sec. 3.3 operation choice: (i) attention, (ii) MLP, (iii) the entire block
        f_x, ref = {"attn": (sa, x), "mlp": (mlp, x_prime), "block": (x_hat, x)}[op]
        score = representation_shift(f_x, ref, dist)                    # Eq. (4)
    return {"x_prime": x_prime, "sa": sa, "mlp": mlp, "x_hat": x_hat, "score": score}


def representation_shift(f_x: np.ndarray, x: np.ndarray, dist: str = "l2") -> np.ndarray:
    """Eq. (4): per token, D(F(x), x) over the channel axis, D one of the distances of
    Sec. 3.3: L2 norm of the difference (the method), L1 norm of the difference, or the
    cosine distance 1 - a.b / (|a| |b|)."""
    a, b = np.asarray(f_x, F64), np.asarray(x, F64)
    if dist == "l2":
        diff = a - b
        return np.sqrt((diff * diff).sum(axis=-1))
    if dist == "l1":
        return np.abs(a - b).sum(axis=-1)
    if dist == "cos":
        dot = (a * b).sum(axis=-1)
        den = np.sqrt((a * a).sum(axis=-1)) * np.sqrt((b * b).sum(axis=-1))
        return 1.0 - dot / np.maximum(den, 1e-8)
    raise ValueError(dist)


# ----------------------------------------------------------------------------- selection

def keep_count(ratio: float, L: int) -> int:
    """Kept tokens when a fraction `ratio` of the current L is kept: floor(r*L + 1/2)."""
    return int(math.floor(float(ratio) * float(L) + 0.5))


def select_kept(scores: Sequence[float], k: int, has_cls: bool) -> List[int]:
    """Indices of the k kept tokens of one sample, ascending.

    Drops the lowest-scoring tokens (Sec. 3.2 toy experiments; Sec. 4): rank by score
    descending, ties to the lower index, NaN below every number, the class token
    (index 0) above everything when present."""
    L = len(scores)
    if not (1 <= k <= L):
        raise ValueError(f"k={k} outside [1, {L}]")

    def rank(i):
        s = float(scores[i])
        forced = 1 if (has_cls and i == 0) else 0
        nan = math.isnan(s)
        return (-forced, nan, 0.0 if nan else -s, i)

    order = sorted(range(L), key=rank)
    return sorted(order[:k])


# ----------------------------------------------------------------------------- encoder

def schedule(depth: int, L: int, prune_layers: Sequence[int], keep_ratios: Sequence[float]):
    """Token count entering each block and the kept count at each prune block."""
    if len(prune_layers) != len(keep_ratios):
        raise ValueError("prune_layers and keep_ratios differ in length")
    lens, ks = [], {}
    cur = L
    for b in range(depth):
        lens.append(cur)
        if b in prune_layers:
            k = keep_count(keep_ratios[list(prune_layers).index(b)], cur)
            ks[b] = k
            cur = k
    return lens, ks, cur


def encoder_forward(x: np.ndarray, blocks: List[Dict[str, np.ndarray]], heads: int,
                    prune_layers: Sequence[int], keep_ratios: Sequence[float], has_cls: bool,
                    eps: float = 1e-6, op: str = "mlp", dist: str = "l2"):
    """Blocks in order on one sample; after each listed block keep the top
    floor(r*L+1/2) tokens by the block's representation shift (the method: MLP, L2) and
    compact the block's output to them.  Returns (out [L_final, C], original ids)."""
    cur = np.asarray(x, F64)
    ids = np.arange(cur.shape[0])
    for b, w in enumerate(blocks):
        r = block_forward(cur, w, heads, eps, op=op, dist=dist)
        cur = r["x_hat"]
        if b in prune_layers:
            k = keep_count(keep_ratios[list(prune_layers).index(b)], cur.shape[0])
            kept = select_kept(r["score"], k, has_cls)
            cur = cur[kept]
            ids = ids[kept]
    return cur, ids


# ----------------------------------------------------------------------------- around the encoder

def patch_embed(images: np.ndarray, w_patch: np.ndarray, b_patch: np.ndarray,
                cls: np.ndarray, pos: np.ndarray, patch: int) -> np.ndarray:
    """Tokens of one sample (Sec. 3.1).  images [T][Cin][H][W] (T = 1 for an image);
    each P x P patch, flattened as (channel, row, column), times w_patch [C][Cin*P*P]
    plus b_patch; patches in raster order within a frame, frames in order; the class
    token `cls` [C] (or None) first; pos [L][C] added to every token."""
    img = np.asarray(images, F64)
    T, cin, H, W = img.shape
    P = int(patch)
    if H % P or W % P:
        raise ValueError("image size must be a multiple of the patch size")
    rows = []
    for t in range(T):
        for pr in range(H // P):
            for pc in range(W // P):
                rows.append(img[t, :, pr * P:(pr + 1) * P, pc * P:(pc + 1) * P].reshape(-1))
    tokens = linear(np.stack(rows), w_patch, b_patch)
    if cls is not None:
        tokens = np.concatenate([np.asarray(cls, F64)[None, :], tokens], axis=0)
    pos = np.asarray(pos, F64)
    if pos.shape != tokens.shape:
        raise ValueError(f"position table {pos.shape} does not match tokens {tokens.shape}")
    return tokens + pos


def head(x: np.ndarray, ln_g: np.ndarray, ln_b: np.ndarray, w_head: np.ndarray,
         b_head: np.ndarray, pool: str, eps: float = 1e-6):
    """Final LayerNorm, pooling and linear head of one sample x [L][C].  pool "cls":
    the normalised row of token 0; "mean": the mean over tokens of the normalised rows.
    Returns (features [C], logits [n_out])."""
    xn = layer_norm(np.asarray(x, F64), ln_g, ln_b, eps)
    if pool == "cls":
        feat = xn[0]
    elif pool == "mean":
        feat = xn.mean(axis=0)
    else:
        raise ValueError(pool)
    return feat, linear(feat[None, :], w_head, b_head)[0]


def vit_forward(images: np.ndarray, emb: Dict[str, np.ndarray], blocks: List[Dict[str, np.ndarray]],
                hd: Dict[str, np.ndarray], heads: int, patch: int, prune_layers: Sequence[int],
                keep_ratios: Sequence[float], has_cls: bool, pool: str, eps: float = 1e-6,
                op: str = "mlp", dist: str = "l2"):
    """The whole forward pass of one sample: patch embedding, the pruned encoder, the
    head.  Returns (features, logits, ids of the encoder's output tokens)."""
    x = patch_embed(images, emb["w_patch"], emb["b_patch"], emb["cls"] if has_cls else None,
                    emb["pos"], patch)
    out, ids = encoder_forward(x, blocks, heads, prune_layers, keep_ratios, has_cls, eps, op, dist)
    feat, logits = head(out, hd["ln_g"], hd["ln_b"], hd["w_head"], hd["b_head"], pool, eps)
    return feat, logits, ids


# ----------------------------------------------------------------------------- work model

def block_macs(L: int, C: int, hidden: int = None) -> int:
    """Multiply-accumulates of one block on L tokens: QKV 3LC^2, attention 2L^2C,
    projection LC^2, MLP 2*L*C*hidden (= 8LC^2 at hidden = 4C).  The L^2C and LC^2
    terms are the O(N^2 C + N C^2) cost named in Sec. 3.1."""
    hidden = 4 * C if hidden is None else hidden
    return 4 * L * C * C + 2 * L * L * C + 2 * L * C * hidden


def encoder_gmacs(depth: int, L: int, C: int, prune_layers, keep_ratios,
                  patches: int = None, patch_in: int = 768) -> float:
    """GMACs of a whole encoder forward under the pruning schedule, plus the patch
    embedding (patches x patch_in x C).  The pages' "GFLOPs" columns are MAC counts."""
    lens, _, _ = schedule(depth, L, prune_layers, keep_ratios)
    total = sum(block_macs(l, C) for l in lens)
    if patches is not None:
        total += patches * patch_in * C
    return total / 1e9

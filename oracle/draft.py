"""Draft Attention mask builder and token reorder -- oracle (test infrastructure only).

Source: "科学家提出视频扩散模型加速方法，在H100实现一倍以上端到端加速"
(163.com article on Draft Attention):

* the latent tokens are reshaped into video form [t, h, w]; the reshaped
  queries and keys are downsampled by average pooling into a low-resolution
  draft attention map (paragraph on the core innovation);
* the draft map yields a sparse mask that keeps only the important
  connections of the full-resolution attention (next paragraph);
* when pool_h x pool_w = block_size, one draft-map entry is one block of a
  block-sparse attention kernel (paragraph on aligning with block-sparse
  attention frameworks);
* a reorder gathers the scattered sparse blocks into a contiguous layout
  (the "Full Map" -> "Reordered Full Map" figure paragraph);
* average pooling beats max pooling at high sparsity, and the method is run
  at 90% sparsity (paragraphs on the design details and the experiments);
  both poolings are provided.

Readings taken where the article leaves a step open (every one is listed in
the design notes of the repository):

* pooling is spatial only, within a frame; Q and K are pooled per head, V
  is not; the grid is padded at the bottom and right up to a multiple of
  the tile; pad tokens are excluded from the mean and from attention;
* the reorder is tile-major: tiles (t, hb, wb) in raster order, and within
  a tile the valid tokens in (hi, wi) raster order first, then the pads;
* the draft map is the unscaled fp32 logit q̄·k̄ (softmax and 1/sqrt(d) are
  monotone in each row and do not change a row's top-k); its arithmetic is
  fixed so that two implementations agree bit for bit: the pool sums the
  valid tokens of a tile one at a time in slot order starting from +0.0
  and divides once by the count, both in IEEE fp32; the score folds
  c = 0..d-1 as acc = fl(acc + fl(q̄[c] * k̄[c])) with no fused multiply-add;
* each query-block row keeps k = clamp(floor((1 - sparsity) * nb + 0.5), 1, nb)
  KV blocks, the largest scores first, the lower block index first on a
  tie, -0 equal to +0; the kept list is stored in ascending block order.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class DraftGrid:
    T: int
    H: int
    W: int  # grid width (tokens per row)
    pool_h: int
    pool_w: int

    @property
    def block_size(self) -> int:
        return self.pool_h * self.pool_w

    @property
    def Hp(self) -> int:
        return -(-self.H // self.pool_h) * self.pool_h

    @property
    def Wp(self) -> int:
        return -(-self.W // self.pool_w) * self.pool_w

    @property
    def nbh(self) -> int:
        return self.Hp // self.pool_h

    @property
    def nbw(self) -> int:
        return self.Wp // self.pool_w

    @property
    def nb(self) -> int:
        return self.T * self.nbh * self.nbw

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def N_pad(self) -> int:
        return self.nb * self.block_size


def draft_grid(T: int, H: int, W: int, pool_h: int, pool_w: int) -> DraftGrid:
    if min(T, H, W, pool_h, pool_w) < 1:
        raise ValueError("grid and pool sizes must be positive")
    return DraftGrid(T, H, W, pool_h, pool_w)


def draft_permutation(g: DraftGrid):
    """Tile-major reorder.

    Returns perm [N_pad] (new position -> original token, -1 for a pad),
    inv_perm [N] (original token -> new position) and block_valid [nb]
    (number of valid tokens, which occupy the first slots of each block)."""
    bs = g.block_size
    perm = np.full(g.N_pad, -1, dtype=np.int32)
    block_valid = np.zeros(g.nb, dtype=np.int32)
    for t in range(g.T):
        for hb in range(g.nbh):
            for wb in range(g.nbw):
                b = (t * g.nbh + hb) * g.nbw + wb
                slot = 0
                for hi in range(g.pool_h):
                    for wi in range(g.pool_w):
                        y = hb * g.pool_h + hi
                        x = wb * g.pool_w + wi
                        if y < g.H and x < g.W:
                            perm[b * bs + slot] = (t * g.H + y) * g.W + x
                            slot += 1
                block_valid[b] = slot
    inv_perm = np.full(g.N, -1, dtype=np.int32)
    valid = perm >= 0
    inv_perm[perm[valid]] = np.nonzero(valid)[0].astype(np.int32)
    return perm, inv_perm, block_valid


def draft_pool(x: np.ndarray, g: DraftGrid, mode: str = "mean") -> np.ndarray:
    """Per-tile fp32 mean (or maximum) of x ([heads, N, d], fp32 values) over valid tokens.

    mean: acc starts at +0.0; the tile's valid tokens are added one at a time
    in slot order, each add rounded to fp32; the mean is one fp32 division.
    max: the largest value over the valid tokens, plus +0.0 (a zero result is
    +0); exact, so the order does not matter."""
    x = np.asarray(x, dtype=np.float32)
    heads, n, d = x.shape
    assert n == g.N
    perm, _, block_valid = draft_permutation(g)
    bs = g.block_size
    if mode == "max":
        if not np.all(np.isfinite(x)):
            raise ValueError("max pooling needs finite inputs")
        out = np.full((heads, g.nb, d), -np.inf, dtype=np.float32)
        pb = perm.reshape(g.nb, bs)
        for b in range(g.nb):
            rows = pb[b, : block_valid[b]]
            out[:, b, :] = x[:, rows, :].max(axis=1)
        return (out + np.float32(0.0)).astype(np.float32)
    if mode != "mean":
        raise ValueError(f"unknown pooling {mode!r}")
    acc = np.zeros((heads, g.nb, d), dtype=np.float32)
    pb = perm.reshape(g.nb, bs)
    for slot in range(bs):
        live = slot < block_valid
        if not live.any():
            continue
        rows = pb[live, slot]
        acc[:, live, :] = acc[:, live, :] + x[:, rows, :]  # fp32 + fp32 -> fp32
    cnt = block_valid.astype(np.float32)[None, :, None]
    return (acc / cnt).astype(np.float32)


def draft_scores(qbar: np.ndarray, kbar: np.ndarray) -> np.ndarray:
    """Draft map s̄[h, i, j] = fold_c fl(acc + fl(q̄[h,i,c] * k̄[h,j,c])), fp32, no FMA."""
    qbar = np.asarray(qbar, dtype=np.float32)
    kbar = np.asarray(kbar, dtype=np.float32)
    heads, nb, d = qbar.shape
    out = np.empty((heads, nb, kbar.shape[1]), dtype=np.float32)
    for h in range(heads):
        acc = np.zeros((nb, kbar.shape[1]), dtype=np.float32)
        for c in range(d):
            prod = np.multiply.outer(qbar[h, :, c], kbar[h, :, c])  # fp32 * fp32 -> fp32
            acc = acc + prod
        out[h] = acc
    return out


def topk_count(sparsity: float, nb: int) -> int:
    """k = clamp(floor((1 - sparsity) * nb + 0.5), 1, nb), in double precision."""
    k = math.floor((1.0 - sparsity) * nb + 0.5)
    return max(1, min(nb, k))


def draft_topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Per row, the k largest scores (lower index first on ties, -0 == +0), ascending."""
    scores = np.asarray(scores, dtype=np.float32)
    if not np.all(np.isfinite(scores)):
        raise ValueError("draft scores must be finite")
    heads, rows, nb = scores.shape
    s = scores + np.float32(0.0)  # -0 + +0 = +0: canonicalise signed zero
    out = np.empty((heads, rows, k), dtype=np.int32)
    idx = np.arange(nb)
    for h in range(heads):
        for i in range(rows):
            order = np.lexsort((idx, -s[h, i].astype(np.float64)))  # score desc, then index asc
            out[h, i] = np.sort(order[:k])
    return out


def draft_mask(q: np.ndarray, k: np.ndarray, g: DraftGrid, sparsity: float, pool: str = "mean"):
    """Full Draft mask builder on fp32 inputs [heads, N, d].

    Returns (kv_idx [heads, nb, k], kv_cnt [heads, nb], qbar, kbar, scores)."""
    qbar = draft_pool(q, g, pool)
    kbar = draft_pool(k, g, pool)
    s = draft_scores(qbar, kbar)
    kk = topk_count(sparsity, g.nb)
    kv_idx = draft_topk(s, kk)
    kv_cnt = np.full(kv_idx.shape[:2], kk, dtype=np.int32)
    return kv_idx, kv_cnt, qbar, kbar, s

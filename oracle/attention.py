"""Softmax attention over explicit key sets in float64 -- oracle (test infrastructure only).

Sources:

* dense self-attention O = softmax(Q Kᵀ / sqrt(d)) V over all N tokens, whose
  cost grows quadratically with the sequence ("LVSA: Training-Free Sparse
  Attention for Long Video Diffusion", technical summary §1 "Problem
  statement");
* frame-block-sparse execution: query frame t attends only to the P tokens
  of each frame in A(t), so the cost is O(T·C·P²·d) (same page, §2,
  "Complexity");
* block-sparse execution of the Draft mask on the reordered tokens, one
  draft-map entry per attention block (Draft Attention article, paragraphs
  on pool_h x pool_w = block_size and on the reorder).

Readings: the softmax scale is 1/sqrt(d) and attention is not causal; a
query row with an empty key set has output 0; pad rows of a reordered
layout (slots at or beyond a block's valid count) are neither queries nor
keys, and their output rows are 0.

All arithmetic here is float64 on the exact input values (bfloat16 bit
patterns are decoded exactly), so the only difference from real arithmetic
is float64 rounding.
"""
from __future__ import annotations

import numpy as np


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 values of an input tensor: uint16 = bfloat16 bits, else float."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def attention_keyset(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """softmax(q kᵀ * scale) v for queries q_rows [m, d] over keys k_sel/v_sel [L, d]."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    if k_sel.shape[0] == 0:
        return np.zeros((q_rows.shape[0], v_sel.shape[1]), dtype=np.float64)
    s = (q_rows @ np.asarray(k_sel, dtype=np.float64).T) * scale
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    return (p @ np.asarray(v_sel, dtype=np.float64)) / p.sum(axis=1, keepdims=True)


def _chunks(rows: np.ndarray, size: int):
    for i in range(0, len(rows), size):
        yield rows[i : i + size]


def dense_attention(q, k, v, scale: float | None = None, rows=None, heads=None, chunk: int = 512,
                    fn=None) -> np.ndarray:
    """Dense attention; q, k, v [heads, N, d] (bf16 bits or float). Returns fp64 [len(heads), len(rows), d].
    fn(q_rows, k_sel, v_sel, scale) evaluates a row set over its keys (default: attention_keyset)."""
    fn = attention_keyset if fn is None else fn
    H, n, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    rows = np.arange(n) if rows is None else np.asarray(rows)
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(heads), len(rows), d), dtype=np.float64)
    for hi, h in enumerate(heads):
        kh, vh = to_f64(k[h]), to_f64(v[h])
        for ci, r in enumerate(_chunks(rows, chunk)):
            out[hi, ci * chunk : ci * chunk + len(r)] = fn(to_f64(q[h, r]), kh, vh, scale)
    return out


def _block_keys(blocks, block_k: int, n: int, block_valid) -> np.ndarray:
    """Concatenated key rows of the listed blocks (valid prefix of each, clipped to n)."""
    parts = []
    for b in blocks:
        lo = int(b) * block_k
        cnt = block_k if block_valid is None else int(block_valid[b])
        hi = min(lo + cnt, n)
        if hi > lo:
            parts.append(np.arange(lo, hi))
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def block_sparse_attention(q, k, v, block_q: int, block_k: int, kv_idx, kv_cnt, mask_heads: int = 1,
                           block_valid=None, scale: float | None = None, rows=None, heads=None,
                           fn=None) -> np.ndarray:
    """Block-sparse attention in the layout given.

    Query row i of head h belongs to query block i // block_q; its keys are
    the valid rows of the KV blocks kv_idx[hm, qb, :kv_cnt[hm, qb]] with
    hm = h if mask_heads > 1 else 0 (each block contributes the rows
    [b*block_k, b*block_k + valid(b)) inside [0, n), valid(b) = block_valid[b]
    or block_k). A query row at a slot >= block_valid of its block is a pad
    and gets output 0. Returns fp64 [len(heads), len(rows), d]. fn evaluates a
    row set over its keys (default: attention_keyset)."""
    fn = attention_keyset if fn is None else fn
    H, n, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    kv_idx = np.asarray(kv_idx)
    kv_cnt = np.asarray(kv_cnt)
    if kv_idx.ndim == 2:
        kv_idx = kv_idx[None]
        kv_cnt = kv_cnt[None]
    rows = np.arange(n) if rows is None else np.asarray(rows)
    heads = list(range(H)) if heads is None else list(heads)
    out = np.zeros((len(heads), len(rows), d), dtype=np.float64)
    qblk = rows // block_q
    for hi, h in enumerate(heads):
        hm = h if mask_heads > 1 else 0
        for qb in np.unique(qblk):
            sel = np.nonzero(qblk == qb)[0]
            r = rows[sel]
            if block_valid is not None:
                live = (r - qb * block_q) < int(block_valid[qb])
                sel, r = sel[live], r[live]
            if len(r) == 0:
                continue
            keys = _block_keys(kv_idx[hm, qb, : int(kv_cnt[hm, qb])], block_k, n, block_valid)
            out[hi, sel] = fn(to_f64(q[h, r]), to_f64(k[h, keys]), to_f64(v[h, keys]), scale)
    return out


def draft_attention_original_order(q, k, v, perm, inv_perm, block_valid, block_size: int, kv_idx, kv_cnt,
                                   scale: float | None = None, heads=None, rows=None, fn=None) -> np.ndarray:
    """Draft block-sparse attention computed directly in the original token order.

    Token n sits in block b = inv_perm[n] // block_size of the reorder; its keys
    are the original tokens perm[b'*block_size + o] for every listed block b'
    and every valid slot o < block_valid[b']. No reordered tensor is built, so
    comparing this with reorder -> block-sparse attention -> inverse reorder
    checks that the reorder does not change the result.
    Returns fp64 [len(heads), len(rows), d] (rows = original token indices,
    default all). fn evaluates a row set over its keys (default:
    attention_keyset)."""
    fn = attention_keyset if fn is None else fn
    H, n, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    heads = list(range(H)) if heads is None else list(heads)
    rows = np.arange(n) if rows is None else np.asarray(rows)
    assert np.all(inv_perm >= 0)
    qblk = np.asarray(inv_perm)[rows] // block_size
    out = np.zeros((len(heads), len(rows), d), dtype=np.float64)
    for hi, h in enumerate(heads):
        for b in np.unique(qblk):
            sel = np.nonzero(qblk == b)[0]
            parts = [perm[bb * block_size : bb * block_size + int(block_valid[bb])] for bb in kv_idx[h, b, : int(kv_cnt[h, b])]]
            keys = np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)  # empty list: no keys
            out[hi, sel] = fn(to_f64(q[h, rows[sel]]), to_f64(k[h, keys]), to_f64(v[h, keys]), scale)
    return out


def attention_statistics(q_rows: np.ndarray, k_all: np.ndarray, keep: np.ndarray, scale: float) -> dict:
    """Statistics of the attention of q_rows [m, d] over all keys k_all [n, d],
    and over the subset the mask keeps (boolean keep [m, n]).

    Per row: the standard deviation of the scaled logits over all keys, the
    entropy (nats) of the dense softmax, the entropy of the softmax restricted
    to the kept keys, and the share of the dense softmax mass that falls on
    the kept keys. Returns each as an array of m values."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    s = (q_rows @ np.asarray(k_all, dtype=np.float64).T) * scale
    std = s.std(axis=1)

    def entropy(logits, live):
        z = np.where(live, logits, -np.inf)
        m = z.max(axis=1, keepdims=True)
        p = np.where(live, np.exp(z - m), 0.0)
        p = p / p.sum(axis=1, keepdims=True)
        return -(p * np.log(np.where(p > 0, p, 1.0))).sum(axis=1), p

    everything = np.ones_like(keep, dtype=bool)
    h_dense, p_dense = entropy(s, everything)
    h_kept, _ = entropy(s, keep)
    mass = (p_dense * keep).sum(axis=1)
    return {"logit_std": std, "entropy_dense": h_dense, "entropy_kept": h_kept, "mass_kept": mass}

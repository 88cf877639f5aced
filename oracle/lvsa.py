"""LVSA attend sets A(t) = G_s ∪ W(t) -- oracle (test infrastructure only).

Source: "LVSA: Training-Free Sparse Attention for Long Video Diffusion",
technical summary §2 "Methodology", "Core mechanism":

* query frame t attends to a set A(t) of frames instead of all of
  {0, ..., T-1}; A(t) is the union of global anchor frames G and a local
  window W(t);
* the anchor set G_s is shifted by the denoising step s modulo T_per, and
  over T_per consecutive steps every frame is an anchor exactly once;
* every frame sees a local temporal window of size W; where the window
  overlaps anchors it is widened so that |A(t)| stays at about the budget C
  (C is normally the model's training length, 21 latent frames for Wan 2.1
  1.3B).

Readings taken where the page leaves a step open:

* anchors are the frames f with f ≡ s (mod T_per) -- spacing T_per, offset
  s mod T_per, which is the only evenly spaced set for which a one-frame
  shift per step makes every frame an anchor exactly once per T_per steps;
* the window is the first k frames in nearest-first order, the order of the
  key (|f - t|, f): centred on t, the earlier frame first on a tie, shifted
  inward at the ends of the video;
* widening adds one frame at a time in that order, starting from k = W,
  until |A(t)| = min(C, T) or every frame is in; an A(t) that already
  exceeds C with k = W is kept whole (anchors and the base window are never
  dropped).
"""
from __future__ import annotations

import numpy as np


def anchors(T: int, T_per: int, s: int) -> list[int]:
    """G_s: the frames f in [0, T) with f ≡ s (mod T_per)."""
    off = s % T_per
    return [f for f in range(T) if f % T_per == off]


def nearest_order(t: int, T: int) -> list[int]:
    """All frames sorted by the key (|f - t|, f): nearest first, earlier on ties."""
    return sorted(range(T), key=lambda f: (abs(f - t), f))


def attend_set(t: int, T: int, C: int, window: int, T_per: int, s: int) -> list[int]:
    """A(t) = G_s ∪ N_k(t), ascending, with k grown from the window size W."""
    if not (0 <= t < T) or C < 1 or window < 1 or T_per < 1:
        raise ValueError("invalid LVSA parameters")
    G = set(anchors(T, T_per, s))
    order = nearest_order(t, T)
    target = min(C, T)
    k = min(window, T)
    A = G | set(order[:k])
    while len(A) < target and k < T:
        k += 1
        A = G | set(order[:k])
    return sorted(A)


def lvsa_capacity(T: int, C: int, window: int, T_per: int, s: int) -> int:
    """Largest |A(t)| over all query frames t."""
    return max(len(attend_set(t, T, C, window, T_per, s)) for t in range(T))


def lvsa_mask(T: int, C: int, window: int, T_per: int, s: int, cap: int | None = None):
    """Frame lists in ELL form: kv_idx [T, cap] int32 ascending, -1 padded; kv_cnt [T]."""
    sets = [attend_set(t, T, C, window, T_per, s) for t in range(T)]
    need = max(len(a) for a in sets)
    if cap is None:
        cap = need
    if cap < need:
        raise ValueError(f"cap {cap} < required {need}")
    kv_idx = np.full((T, cap), -1, dtype=np.int32)
    kv_cnt = np.zeros(T, dtype=np.int32)
    for t, a in enumerate(sets):
        kv_idx[t, : len(a)] = a
        kv_cnt[t] = len(a)
    return kv_idx, kv_cnt

"""Seeded synthetic inputs for video-DiT attention workloads.

This module only *creates* tensors: it holds none of the attention, mask or
pooling arithmetic. Both the CPU oracle's tests and the HIP path's tests and
benchmark draw their inputs from here, so the two sides see the same bytes.

Two generators:

* ``iid_qkv``   -- Q, K, V iid N(0, 1), fp32 (the tiny CPU-checkable case).
* ``video_qkv`` -- Q and K share a smooth low-rank field over the [t, h, w]
  token grid (a sum of 8 random separable sinusoids per head) plus
  0.5 * N(0, 1) noise; V is iid N(0, 1). Values are rounded to bfloat16
  (round to nearest, ties to even) and returned as uint16 bit patterns.

Token order is frame-major: n = (t * H + y) * W + x, matching the [t, h, w]
reshape that both pages build on (Draft Attention article, paragraph on
reshaping latent tokens into video form; LVSA technical summary §2, the
frame set {0, ..., T-1}).

Seeding: ``SeedSequence(seed)`` spawns four children [field, q-noise,
k-noise, v]; each child spawns one grandchild per head, so any single head
can be regenerated on its own.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_to_f32",
    "iid_qkv",
    "video_qkv",
    "video_qkv_head",
    "head_streams",
    "Workload",
    "WORKLOADS",
]

N_SINUSOIDS = 8
NOISE_STD = 0.5


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction (no NaN handling needed here)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact fp32 values."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def head_streams(seed: int, heads: int):
    """Per-head numpy Generators for [field, q-noise, k-noise, v]."""
    kids = np.random.SeedSequence(seed).spawn(4)
    return [[np.random.Generator(np.random.PCG64(g)) for g in k.spawn(heads)] for k in kids]


def iid_qkv(seed: int, heads: int, n: int, d: int):
    """Q, K, V iid N(0,1) as fp32 arrays of shape [heads, n, d]."""
    streams = head_streams(seed, heads)
    out = []
    for which in (1, 2, 3):
        arr = np.empty((heads, n, d), dtype=np.float32)
        for h in range(heads):
            arr[h] = streams[which][h].standard_normal((n, d), dtype=np.float32)
        out.append(arr)
    return tuple(out)


def _field(rng: np.random.Generator, T: int, H: int, W: int, d: int) -> np.ndarray:
    """Smooth low-rank field F(t, y, x) in R^d, shape [T*H*W, d], fp32.

    F = sum_j sin(wt*t + pt) * sin(wh*y + ph) * sin(ww*x + pw) * u_j with
    frequencies ~ U(0, pi/4) rad per frame/token, phases ~ U(0, 2*pi) and
    loadings u_j ~ N(0, I_d)."""
    om = rng.uniform(0.0, np.pi / 4.0, size=(N_SINUSOIDS, 3))
    ph = rng.uniform(0.0, 2.0 * np.pi, size=(N_SINUSOIDS, 3))
    u = rng.standard_normal((N_SINUSOIDS, d))
    st = np.sin(om[:, 0:1] * np.arange(T)[None, :] + ph[:, 0:1])  # [8, T]
    sy = np.sin(om[:, 1:2] * np.arange(H)[None, :] + ph[:, 1:2])  # [8, H]
    sx = np.sin(om[:, 2:3] * np.arange(W)[None, :] + ph[:, 2:3])  # [8, W]
    # A[n, j] = st[j, t] * sy[j, y] * sx[j, x], n = (t*H + y)*W + x
    a = (st.T[:, None, None, :] * sy.T[None, :, None, :] * sx.T[None, None, :, :]).reshape(T * H * W, N_SINUSOIDS)
    return (a @ u).astype(np.float32)


def video_qkv_head(seed: int, h: int, heads: int, T: int, H: int, W: int, d: int, streams=None):
    """One head of the video-shaped workload: (q, k, v) bf16 bits [T*H*W, d]."""
    if streams is None:
        streams = head_streams(seed, heads)
    n = T * H * W
    f = _field(streams[0][h], T, H, W, d)
    q = f + np.float32(NOISE_STD) * streams[1][h].standard_normal((n, d), dtype=np.float32)
    q = bf16_round(q)
    k = f + np.float32(NOISE_STD) * streams[2][h].standard_normal((n, d), dtype=np.float32)
    k = bf16_round(k)
    v = bf16_round(streams[3][h].standard_normal((n, d), dtype=np.float32))
    return q, k, v


def video_qkv(seed: int, heads: int, T: int, H: int, W: int, d: int, threads: int | None = None):
    """All heads: (q, k, v) as uint16 bf16 bits of shape [heads, T*H*W, d]."""
    n = T * H * W
    q = np.empty((heads, n, d), dtype=np.uint16)
    k = np.empty_like(q)
    v = np.empty_like(q)
    streams = head_streams(seed, heads)

    def one(h):
        q[h], k[h], v[h] = video_qkv_head(seed, h, heads, T, H, W, d, streams)

    if threads is None:
        threads = min(16, max(1, len(os.sched_getaffinity(0))))
    with _cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(one, range(heads)))
    return q, k, v


@dataclass(frozen=True)
class Workload:
    """Shape and mask parameters of one attention workload."""

    name: str
    T: int
    H: int
    W: int
    heads: int
    d: int
    dtype: str  # "f32" or "bf16"
    kind: str  # "lvsa" or "draft"
    seed: int
    C: int = 0
    window: int = 0
    T_per: int = 1
    pool_h: int = 0
    pool_w: int = 0
    sparsity: float = 0.0

    @property
    def P(self) -> int:
        return self.H * self.W

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


# The five workloads: a tiny CPU-checkable grid, Wan-2.1-1.3B at training
# length (T = 21 latent frames of 30x52 tokens, 12 heads, d = 128) and at 6x
# length (T = 126), HunyuanVideo-shaped Draft Attention (T = 33 frames of
# 45x80 tokens, 24 heads, 8x16 pooling, 90% sparsity), Wan-2.1-14B at 6x
# length (40 heads), and LVSA on a HunyuanVideo-shaped grid at 2x its
# training length (257 video frames = 65 latent frames, budget C = 33 latent
# frames = the 129-frame training length).
WORKLOADS = {
    "tiny": Workload("tiny", T=4, H=8, W=8, heads=2, d=64, dtype="f32", kind="lvsa", seed=1,
                     C=3, window=2, T_per=2),
    "wan1.3b-1x": Workload("wan1.3b-1x", T=21, H=30, W=52, heads=12, d=128, dtype="bf16", kind="lvsa",
                           seed=2, C=21, window=5, T_per=8),
    "wan1.3b-6x": Workload("wan1.3b-6x", T=126, H=30, W=52, heads=12, d=128, dtype="bf16", kind="lvsa",
                           seed=3, C=21, window=5, T_per=8),
    "hunyuan-draft": Workload("hunyuan-draft", T=33, H=45, W=80, heads=24, d=128, dtype="bf16", kind="draft",
                              seed=4, pool_h=8, pool_w=16, sparsity=0.9),
    "wan14b-6x": Workload("wan14b-6x", T=126, H=30, W=52, heads=40, d=128, dtype="bf16", kind="lvsa",
                          seed=5, C=21, window=5, T_per=8),
    "hunyuan-lvsa-2x": Workload("hunyuan-lvsa-2x", T=65, H=45, W=80, heads=24, d=128, dtype="bf16", kind="lvsa",
                                seed=6, C=33, window=5, T_per=8),
    "hunyuan-lvsa-1.5x": Workload("hunyuan-lvsa-1.5x", T=49, H=45, W=80, heads=24, d=128, dtype="bf16",
                                  kind="lvsa", seed=7, C=33, window=5, T_per=8),
}

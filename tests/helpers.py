"""Shared helpers for the GPU parity tests (host-side marshalling and comparisons)."""
import sys

import numpy as np

# Attention tolerance for bf16 inputs with fp32 accumulation, against fp64.
MAX_ABS = 1e-2
REL_L2 = 5e-3


def note(msg: str):
    """Name the case about to run on the GPU (flushed, so a crash leaves it behind)."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_dev_bf16(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def to_dev(a: np.ndarray):
    import torch

    if a.dtype == np.uint16:
        return to_dev_bf16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def attn_errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(got - ref)
    max_abs = float(err.max()) if err.size else 0.0
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nref) if nref > 0 else float(np.linalg.norm(got - ref))
    return max_abs, rel


def assert_attn_close(got, ref, max_abs=MAX_ABS, rel_l2=REL_L2, what=""):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    m, r = attn_errors(got, ref)
    assert m <= max_abs and r <= rel_l2, f"{what}: max-abs {m:.3e} (bound {max_abs}), rel-L2 {r:.3e} (bound {rel_l2})"
    return m, r


def sample_frame_rows(rng, T: int, P: int, nframes: int = 6, per_frame: int = 96):
    """Query rows for sampled parity at full size: the first, second, middle and
    last frames plus random ones; in each, the first 32 rows, the last 32 rows
    (the ragged tail of a frame) and random rows."""
    frames = sorted(set([0, 1, T // 2, T - 1] + list(rng.choice(T, size=max(0, nframes - 4), replace=False))))
    rows = []
    for f in frames:
        base = f * P
        loc = set(range(min(32, P))) | set(range(max(0, P - 32), P))
        loc |= set(rng.choice(P, size=min(P, max(0, per_frame - len(loc))), replace=False).tolist())
        rows.extend(base + np.array(sorted(loc)))
    return np.array(rows, dtype=np.int64)


# Per-tile offsets (one per 64-key tile) added to one channel of K, so that
# scores jump by up to ~30 bits (base 2) from one tile of the key walk to the
# next: the attention kernels then move their running reference, rescale O
# and recompute the tile on many tiles, for some rows of a wave and not for
# others (the rows weigh the channel differently).
TILE_OFFSETS = {
    "rising": lambda nt: 25.0 * np.arange(nt),
    "zigzag": lambda nt: np.resize(np.array([0, 40, 10, 90, 95, 30, 160, 20, 161, 200, 5, 240], np.float64), nt),
    "falling": lambda nt: 25.0 * (nt - 1 - np.arange(nt)),
}


def jumping_scores_qkv(seed: int, heads: int, ntile: int, d: int, pattern: str):
    """fp32 Q, K, V [heads, 64*ntile, d]: N(0, 1) plus Q[:, :, 0] = 8 u (u
    uniform in [0.05, 1] per row) and K[:, :, 0] += the offset of the key's
    64-key tile."""
    rng = np.random.default_rng(seed)
    n = 64 * ntile
    q, k, v = (rng.standard_normal((heads, n, d)).astype(np.float32) for _ in range(3))
    q[:, :, 0] = 8.0 * rng.uniform(0.05, 1.0, size=(heads, n)).astype(np.float32)
    k[:, :, 0] += np.repeat(TILE_OFFSETS[pattern](ntile), 64).astype(np.float32)[None, :]
    return q, k, v


def bf16_decode_fields(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float64 from the format's field definition
    (1 sign bit, 8 exponent bits with bias 127, 7 fraction bits; exponent 0
    is zero or subnormal with scale 2^-126, exponent 255 is infinity or NaN),
    computed with integer fields and ldexp rather than a bit shift, so it
    checks the oracle's decode by a different route."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = (b & 0x7F).astype(np.float64)
    normal = np.ldexp(1.0 + m / 128.0, (e - 127).astype(np.int32))
    sub = np.ldexp(m / 128.0, -126)
    special = np.where(m == 0, np.inf, np.nan)
    mag = np.where(e == 0, sub, np.where(e == 255, special, normal))
    return sign * mag

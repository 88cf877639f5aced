"""FP8 (OCP E4M3) quantization for the low-precision attention variant --
oracle (test infrastructure only).

Source: the Draft Attention article (163.com) names quantization as the next
step after the sparse mask; the pages fix no format, granularity or
rounding. Readings taken here (listed in the design notes):

* format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits (bias 7), 3
  mantissa bits, subnormals down to 2^-9, largest finite 448, no infinity;
* one scale per (tensor, head): scale = fl32(amax / 448) with amax the
  largest |x| over the head (scale = 1 when amax = 0), so the largest value
  maps to 448;
* byte = e4m3 nearest to fl32(x / scale) (IEEE fp32 division), ties to the
  even mantissa, the fp32 quotient first clamped to [-448, 448]; -0 stays -0;
* the dequantized value is decode(byte) * scale, computed exactly.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """Value of every byte 0..255 (NaN for the two NaN codes 0x7F, 0xFF), from
    the format definition: (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, and
    (-1)^s * 2^-6 * (m/8) for e = 0."""
    out = np.empty(256, dtype=np.float64)
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        e = (b >> 3) & 0xF
        m = b & 0x7
        if e == 0xF and m == 0x7:
            out[b] = np.nan
        elif e == 0:
            out[b] = s * 2.0 ** -6 * (m / 8.0)
        else:
            out[b] = s * 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return out


_TABLE = e4m3_decode_table()
# non-negative finite codes in increasing value (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALS = _TABLE[:0x7F]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round fp32 values (|x| <= 448 after the caller's clamp) to the nearest
    E4M3 code, ties to the code with the even mantissa (the even code)."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("e4m3_encode expects finite values within [-448, 448]")
    hi = np.searchsorted(_POS_VALS, a, side="left")      # first code with value >= a
    hi = np.clip(hi, 0, len(_POS_VALS) - 1)
    lo = np.clip(hi - 1, 0, len(_POS_VALS) - 1)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(take_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a == _POS_VALS[hi], _POS_CODES[hi], code)
    sign = np.signbit(x).astype(np.int64) << 7
    return (code | sign).astype(np.uint8)


def quantize_per_head(x: np.ndarray, transpose: bool = False):
    """x: [heads, n, d] values exactly representable in fp32 (bf16 or fp32 inputs).
    Returns (codes uint8 [heads, n, d] or [heads, d, n], scales fp32 [heads])."""
    x = np.asarray(x, dtype=np.float32)
    heads = x.shape[0]
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(heads, dtype=np.float32)
    for h in range(heads):
        amax = np.float32(np.max(np.abs(x[h]))) if x[h].size else np.float32(0)
        s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
        q = (x[h] / s).astype(np.float32)  # IEEE fp32 division
        q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
        codes[h] = e4m3_encode(q)
        scales[h] = s
    if transpose:
        codes = np.ascontiguousarray(codes.transpose(0, 2, 1))
    return codes, scales


def dequantize(codes: np.ndarray, scales: np.ndarray, transposed: bool = False) -> np.ndarray:
    """Exact fp64 values decode(code) * scale; returns [heads, n, d]."""
    c = np.asarray(codes)
    if transposed:
        c = c.transpose(0, 2, 1)
    return _TABLE[c] * np.asarray(scales, dtype=np.float64)[:, None, None]


def attention_p_e4m3(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention with the probabilities rounded to E4M3 for the PV
    product: p_j = exp(s_j - max_k s_k), O = sum_j e4m3(p_j) v_j / sum_j p_j
    (the row sum over the unrounded p). The plain statement of the FP8
    attention's arithmetic, with the row maximum as the reference; a kernel
    that takes another reference score r (x_j - r <= 8 in base 2) rounds other
    values and differs from this by at most twice p_rounding_bound. Same
    arguments as attention.attention_keyset; returns fp64 [m, d]."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_sel = np.asarray(k_sel, dtype=np.float64)
    v_sel = np.asarray(v_sel, dtype=np.float64)
    if k_sel.shape[0] == 0:
        return np.zeros((q_rows.shape[0], v_sel.shape[1]), dtype=np.float64)
    s = (q_rows @ k_sel.T) * scale
    p = np.exp(s - s.max(axis=1, keepdims=True))
    pr = _TABLE[e4m3_encode(p.astype(np.float32))]
    return (pr @ v_sel) / p.sum(axis=1, keepdims=True)


def p_rounding_bound(q_rows: np.ndarray, k_sel: np.ndarray, v_sel: np.ndarray, scale: float) -> np.ndarray:
    """Per-element bound on |O~ - O| for softmax attention whose probabilities
    are rounded to E4M3 (nearest) before the PV product while the row sum
    keeps the unrounded values; everything else exact. Same arguments as
    attention.attention_keyset (values, not codes); returns fp64 [m, d].

    Derivation (the reading this library takes for its FP8 attention): the
    probabilities are p_j = 2^(x_j - r) with x_j the base-2 scores and r one
    of the row's scores, r <= max_j x_j and x_j - r <= 8, so p_j <= 2^8 < 448
    and max_j p_j >= 1. Rounding to E4M3 moves p by at most 2^-4 p in the
    normal range (p >= 2^-6: 3 mantissa bits), by at most 2^-10 in the
    subnormal range (step 2^-9), and by at most p itself (p < 2^-10 rounds
    to 0): |p~ - p| <= 2^-4 p + min(p, 2^-10). With w the softmax weights,
    p_j = w_j sum_k p_k, and sum_k p_k >= 1 / w_max (since max_j p_j >= 1):
        |O~_c - O_c| <= sum_j |p~_j - p_j| |v_jc| / sum_k p_k
                     <= 2^-4 sum_j w_j |v_jc| + sum_j min(w_j, 2^-10 w_max) |v_jc|."""
    q_rows = np.asarray(q_rows, dtype=np.float64)
    k_sel = np.asarray(k_sel, dtype=np.float64)
    v_abs = np.abs(np.asarray(v_sel, dtype=np.float64))
    if k_sel.shape[0] == 0:
        return np.zeros((q_rows.shape[0], v_abs.shape[1]), dtype=np.float64)
    s = (q_rows @ k_sel.T) * scale
    e = np.exp(s - s.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    small = np.minimum(w, 2.0 ** -10 * w.max(axis=1, keepdims=True))
    return 2.0 ** -4 * (w @ v_abs) + small @ v_abs

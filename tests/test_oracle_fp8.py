"""Pins for the FP8 (OCP E4M3) quantization oracle: format values from the
definition, round-trip, ties to even, brute-force nearest, per-head scales."""
import numpy as np
import pytest

import oracle


def test_decode_table_known_values():
    t = oracle.e4m3_decode_table()
    known = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0,
             0x3F: 1.875, 0x40: 2.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for b, v in known.items():
        assert t[b] == v, hex(b)
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)                      # 127 increasing non-negative codes
    assert np.array_equal(t[0x80:0xFF], -pos)            # sign bit negates
    assert len(np.unique(pos)) == 127


def test_encode_round_trip_and_ties_to_even():
    t = oracle.e4m3_decode_table()
    codes = np.array([b for b in range(256) if not np.isnan(t[b])], dtype=np.uint8)
    vals = t[codes].astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    pos = t[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # exact in fp32 (one more bit than e4m3)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)
    got = oracle.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got.astype(np.int64), want)
    assert np.array_equal(oracle.e4m3_encode(-mids).astype(np.int64), want | 0x80)


def test_encode_brute_force_nearest():
    t = oracle.e4m3_decode_table()
    pos = t[:0x7F]
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.uniform(-448, 448, 3000), rng.standard_normal(3000) * 0.05,
                        rng.standard_normal(2000) * 2.0 ** -8]).astype(np.float32)
    got = oracle.e4m3_encode(x)
    for xi, gi in zip(x, got):
        a = abs(float(xi))
        d = np.abs(pos - a)
        best = np.nonzero(d == d.min())[0]
        code = best[0] if len(best) == 1 else [c for c in best if c % 2 == 0][0]
        assert gi == (code | (0x80 if np.signbit(xi) else 0)), (xi, hex(gi), hex(code))
    with pytest.raises(ValueError):
        oracle.e4m3_encode(np.array([449.0], np.float32))


def test_quantize_per_head_scales_and_layout():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 50, 16)).astype(np.float32)
    x[1] *= 100.0
    x[2] = 0.0
    codes, s = oracle.quantize_per_head(x)
    amax = np.abs(x).max(axis=(1, 2))
    assert s[0] == np.float32(amax[0] / np.float32(448)) and s[1] == np.float32(amax[1] / np.float32(448))
    assert s[2] == 1.0 and np.all(codes[2] == 0)
    for h in (0, 1):  # the largest |x| of a head maps to +-448
        i = np.unravel_index(np.argmax(np.abs(x[h])), x[h].shape)
        assert codes[h][i] & 0x7F == 0x7E
    deq = oracle.dequantize(codes, s)
    rel = np.abs(deq[:2] - x[:2]) / np.maximum(np.abs(x[:2]), s[:2, None, None] * 2.0 ** -6)
    assert rel.max() <= 2.0 ** -4 * 1.0001                 # half an e4m3 ulp relative (normal range)
    ct, st = oracle.quantize_per_head(x, transpose=True)
    assert ct.shape == (3, 16, 50) and np.array_equal(ct.transpose(0, 2, 1), codes) and np.array_equal(st, s)
    assert np.array_equal(oracle.dequantize(ct, st, transposed=True), deq)


def test_quantize_bf16_inputs_exact_division():
    # codes of x/s where x/s is exactly representable: x = s * value
    s = np.float32(0.25)
    vals = oracle.e4m3_decode_table()[[0x38, 0x40, 0x3C, 0x10, 0x7E]].astype(np.float32)  # 1, 2, 1.5, 2^-5, 448
    x = (vals * s)[None, :, None].astype(np.float32)
    codes, sc = oracle.quantize_per_head(x)
    assert sc[0] == np.float32(448 * 0.25 / 448)
    assert list(codes[0, :, 0]) == [0x38, 0x40, 0x3C, 0x10, 0x7E]


def _rounded_p_attention(q_rows, k_sel, v_sel, scale, shift):
    """Attention with p = 2^(x - r) rounded to E4M3 for the PV product and the
    unrounded row sum, r = (row max of the base-2 scores) - shift."""
    t = oracle.e4m3_decode_table()
    x = (np.asarray(q_rows, np.float64) @ np.asarray(k_sel, np.float64).T) * scale / np.log(2.0)
    r = x.max(axis=1, keepdims=True) - shift
    p = np.exp2(x - r)
    pr = t[oracle.e4m3_encode(p.astype(np.float32))].astype(np.float64)
    return (pr @ np.asarray(v_sel, np.float64)) / p.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("seed,L,sc", [(0, 64, 1.0), (1, 700, 3.0), (2, 300, 0.2), (3, 2000, 6.0)])
def test_p_rounding_bound_holds(seed, L, sc):
    """The bound is never exceeded by attention with E4M3-rounded
    probabilities, for reference scores anywhere in [max - 8, max]."""
    rng = np.random.default_rng(seed)
    d = 16
    q = rng.standard_normal((40, d)) * sc
    k = rng.standard_normal((L, d))
    v = rng.standard_normal((L, d)) * rng.uniform(0.1, 3.0, size=(1, d))
    scale = 1.0 / np.sqrt(d)
    exact = oracle.attention_keyset(q, k, v, scale)
    bound = oracle.p_rounding_bound(q, k, v, scale)
    assert bound.shape == exact.shape and np.all(bound > 0)
    worst = 0.0
    for shift in (0.0, 0.37, 3.9, 7.99):
        # shift > 0 is only valid when no score sits more than 8 above r
        got = _rounded_p_attention(q, k, v, scale, shift)
        err = np.abs(got - exact)
        assert np.all(err <= bound * (1 + 1e-9) + 1e-15), (shift, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
    assert worst > 0.05  # the bound is not vacuous on random data


def test_p_rounding_bound_is_tight():
    """Two keys with probabilities 1 and 1.0625 (a tie between E4M3 1 and
    1.125, rounded to the even 1): the error is 2^-4 / 2.0625; the bound
    charges 2^-4 of the unrounded 1.0625 plus the subnormal term, within 8%."""
    q = np.array([[1.0]])
    k = np.array([[0.0], [np.log(1.0625)]])
    v = np.array([[0.0], [1.0]])
    exact = oracle.attention_keyset(q, k, v, 1.0)
    got = _rounded_p_attention(q, k, v, 1.0, np.log2(1.0625))  # r = the first key's score
    err = abs(float(got[0, 0] - exact[0, 0]))
    assert err == pytest.approx(0.0625 / 2.0625, rel=1e-12)
    b = float(oracle.p_rounding_bound(q, k, v, 1.0)[0, 0])
    assert b == pytest.approx(2.0 ** -4 * 1.0625 / 2.0625 + 2.0 ** -10 * 1.0625 / 2.0625, rel=1e-12)
    assert err <= b <= 1.08 * err


def test_p_rounding_bound_subnormal_term():
    """Many keys far below the reference: their probabilities fall in the
    E4M3 subnormal range, where the error is absolute (up to 2^-10 each)."""
    L = 4000
    q = np.array([[1.0]])
    x = np.full(L, -7.3)          # base-2 score relative to the top key: p = 2^-7.3 (subnormal)
    x[0] = 0.0
    k = (x * np.log(2.0))[:, None]
    v = np.ones((L, 1))
    exact = oracle.attention_keyset(q, k, v, 1.0)
    got = _rounded_p_attention(q, k, v, 1.0, 0.0)
    err = abs(float(got[0, 0] - exact[0, 0]))
    b = float(oracle.p_rounding_bound(q, k, v, 1.0)[0, 0])
    p = 2.0 ** -7.3
    t = oracle.e4m3_decode_table()
    assert err == pytest.approx((L - 1) * abs(t[oracle.e4m3_encode(np.float32(p)[None])][0] - p) / (1 + (L - 1) * p),
                                rel=1e-6)
    assert err <= b
    # without the subnormal term the bound would fail here
    w = np.exp2(x) / np.exp2(x).sum()
    assert err > 2.0 ** -4 * float(w @ np.abs(v[:, 0]))


def test_p_rounding_bound_underflow_term():
    """Keys 12 below the top (p = 2^-12 < 2^-10) round to 0: each error is p
    itself, which the bound charges exactly (min(w_j, 2^-10 w_max) = w_j)."""
    L = 4000
    q = np.array([[1.0]])
    x = np.full(L, -12.0)
    x[0] = 0.0
    k = (x * np.log(2.0))[:, None]
    v = np.ones((L, 1))
    v[0] = 0.0
    exact = oracle.attention_keyset(q, k, v, 1.0)
    got = _rounded_p_attention(q, k, v, 1.0, 0.0)
    err = abs(float(got[0, 0] - exact[0, 0]))
    tot = 1 + (L - 1) * 2.0 ** -12
    assert err == pytest.approx((L - 1) * 2.0 ** -12 / tot, rel=1e-9)
    b = float(oracle.p_rounding_bound(q, k, v, 1.0)[0, 0])
    assert err <= b <= err * (1 + 2.0 ** -4) * (1 + 1e-9)


def test_attention_p_e4m3_worked_examples():
    """Hand-computed cases of the FP8 probability rounding."""
    q = np.array([[1.0]])
    # p = (1, 1.0625): 1.0625 is the tie between 1 and 1.125 -> 1 (even)
    k = np.array([[0.0], [np.log(1.0625)]])
    v = np.array([[2.0, 0.0], [1.0, -3.0]])
    got = oracle.attention_p_e4m3(q, k, v, 1.0)
    # reference is the row max (second key): p = (1/1.0625, 1); 1/1.0625 = 0.941..
    # rounds to 0.9375 (E4M3 neighbours 0.9375, 1.0)
    p0 = 1 / 1.0625
    assert np.allclose(got, (0.9375 * v[0] + 1.0 * v[1]) / (p0 + 1.0), rtol=1e-13, atol=0)
    # keys 12 below the top vanish (2^-12 rounds to 0) but stay in the row sum
    L = 100
    x = np.full(L, -12.0)
    x[3] = 0.0
    k = (x * np.log(2.0))[:, None]
    v = np.arange(L, dtype=np.float64)[:, None]
    got = oracle.attention_p_e4m3(q, k, v, 1.0)
    assert got[0, 0] == pytest.approx(3.0 / (1 + (L - 1) * 2.0 ** -12), rel=1e-13)


def test_attention_p_e4m3_exact_when_p_is_representable():
    """Base-2 score gaps that are whole numbers >= -9 give probabilities that
    are powers of two, all E4M3 values: the result is exact attention."""
    rng = np.random.default_rng(3)
    L, d = 50, 8
    x = -rng.integers(0, 10, size=L).astype(np.float64)
    x[0] = 0.0
    q = np.array([[1.0]])
    k = (x * np.log(2.0))[:, None]
    v = rng.standard_normal((L, d))
    assert np.allclose(oracle.attention_p_e4m3(q, k, v, 1.0), oracle.attention_keyset(q, k, v, 1.0),
                       rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1])
def test_attention_p_e4m3_within_bound(seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((30, 16)) * 3
    k = rng.standard_normal((500, 16))
    v = rng.standard_normal((500, 16))
    exact = oracle.attention_keyset(q, k, v, 0.25)
    got = oracle.attention_p_e4m3(q, k, v, 0.25)
    assert np.all(np.abs(got - exact) <= oracle.p_rounding_bound(q, k, v, 0.25))
    assert np.any(got != exact)

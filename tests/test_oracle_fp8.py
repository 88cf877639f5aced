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

"""Pins for the oracle's bfloat16 decode (every bf16 parity case runs its
inputs through it): bit patterns whose values the format fixes, a decoder
written from the field definition, and torch's own bfloat16 conversion."""
import math

import numpy as np
import torch

import oracle
from helpers import bf16_decode_fields

# (bits, value) fixed by the format: 1 sign, 8 exponent (bias 127), 7 fraction bits
FIXED = [
    (0x3F80, 1.0),
    (0xBF80, -1.0),
    (0xC000, -2.0),
    (0x4040, 3.0),
    (0x3F00, 0.5),
    (0x3FC0, 1.5),
    (0x3F81, 1.0 + 2.0 ** -7),
    (0x0000, 0.0),
    (0x0080, 2.0 ** -126),             # smallest normal
    (0x0001, 2.0 ** -133),             # smallest subnormal
    (0x007F, 127 * 2.0 ** -133),       # largest subnormal
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),  # largest finite
    (0xFF7F, -(2.0 - 2.0 ** -7) * 2.0 ** 127),
    (0x4780, 65536.0),
    (0x3DCD, 0.10009765625),           # bf16 nearest to 0.1
]


def test_fixed_patterns():
    bits = np.array([b for b, _ in FIXED], dtype=np.uint16)
    got = oracle.to_f64(bits)
    assert got.dtype == np.float64
    for (b, want), g in zip(FIXED, got):
        assert g == want, f"0x{b:04X}: {g!r} != {want!r}"


def test_signed_zero_and_specials():
    got = oracle.to_f64(np.array([0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) == -1.0
    assert got[1] == math.inf and got[2] == -math.inf
    assert np.isnan(got[3]) and np.isnan(got[4])


def test_every_code_against_field_decoder():
    """All 65536 patterns against the field definition (NaNs as NaN)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits)
    want = bf16_decode_fields(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # signs of zeros too
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))


def test_random_codes_against_torch():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    got = oracle.to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(t)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], t[~nan])


def test_shape_and_float_inputs_pass_through():
    x = np.arange(12, dtype=np.uint16).reshape(3, 4) + np.uint16(0x3F80)
    assert oracle.to_f64(x).shape == (3, 4)
    f = np.array([0.1, -2.5], dtype=np.float32)
    assert np.array_equal(oracle.to_f64(f), f.astype(np.float64))

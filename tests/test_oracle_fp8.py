"""Pins for the FP8 (E4M3) oracle (CPU only): code values that follow from the format's definition,
round trips, ties, saturation, and a brute-force nearest-code check."""
import math

import numpy as np
import pytest

from oracle import fp8 as F


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),       # subnormals: m/8 * 2^-6
    (0x08, 2.0 ** -6), (0x0F, 1.875 * 2.0 ** -6),                # smallest normal binade
    (0x38, 1.0), (0x39, 1.125), (0x3F, 1.875), (0x40, 2.0),      # exponent field 7 = 2^0
    (0x77, 240.0), (0x78, 256.0), (0x7E, 448.0),                 # top binade; 448 is the largest
    (0x80, -0.0), (0xB8, -1.0), (0xFE, -448.0),
])
def test_code_values_follow_the_format(code, value):
    got = float(F.decode(np.array([code], np.uint8))[0])
    assert got == value and math.copysign(1.0, got) == math.copysign(1.0, value)


def test_nan_codes_and_no_infinities():
    d = F.decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(d[0x7F]) and np.isnan(d[0xFF])
    assert np.isnan(d).sum() == 2 and not np.isinf(d).any()
    assert np.nanmax(np.abs(d)) == 448.0


def test_codes_of_one_sign_increase_with_magnitude():
    d = F.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(d) > 0)
    assert np.array_equal(F.decode(np.arange(0x80, 0xFF, dtype=np.uint8)), -d)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.encode(F.decode(codes)), codes)


def test_midpoints_go_to_the_even_code():
    d = F.decode(np.arange(0x7F, dtype=np.uint8))
    mids = (d[:-1] + d[1:]) / 2
    got = F.encode(mids).astype(int)
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F))
    assert np.array_equal(got, want)
    assert np.array_equal(F.encode(-mids).astype(int), want | 0x80)


def test_saturation_and_nan():
    assert list(F.encode(np.array([448.0, 449.0, 470.0, 1e6, np.inf, -1e6, -np.inf]))) == \
        [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert F.encode(np.array([np.nan]))[0] & 0x7F == 0x7F


def test_encode_picks_the_nearest_code_brute_force():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000) * 10.0, rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000),
                        rng.uniform(-460, 460, 1000)])
    got = F.decode(F.encode(x))
    table = F.decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8))
    best = np.min(np.abs(np.minimum(np.abs(x), 448.0)[:, None] * np.sign(x)[:, None] - table[None, :]), axis=1)
    assert np.all(np.abs(got - np.clip(x, -448.0, 448.0)) == best)


def test_quantize_divides_in_float32_then_encodes():
    x = np.array([1.0, 3.0, -7.5, 100.0], np.float32)
    s = np.float32(0.3)
    want = F.encode((x / s).astype(np.float64))
    assert np.array_equal(F.quantize(x, 0.3), want)
    assert np.array_equal(F.dequantize(np.array([0x38, 0xB8], np.uint8), 0.5), [0.5, -0.5])

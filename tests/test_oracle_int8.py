"""Pins of the oracle's INT8 per-token absmax codec (mlxcel "TurboQuant KV
cache", "Available modes": int8, per-token INT8 absmax, about 2x)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _exact_code(x, a):
    """round(127 x / a) with ties to even, in exact rational arithmetic."""
    v = Fraction(127) * Fraction(float(x)) / Fraction(float(a))
    k = v.numerator // v.denominator          # floor
    r = v - k
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k


def test_hand_row():
    # a = 4, scale = 4/127: 1 -> 31.75 -> 32, -2.25 -> -71.4375 -> -71,
    # 0.5 -> 15.875 -> 16, 4 -> 127 (none near a tie)
    x = np.array([[1.0, -2.25, 0.5, 4.0]], np.float16)
    c, s = oracle.int8_quantize(x)
    assert s.dtype == np.float32 and s[0] == np.float32(4.0) / np.float32(127.0)
    assert c.tolist() == [[32, -71, 16, 127]]
    assert np.allclose(oracle.int8_dequantize(c, s)[0], np.array([32, -71, 16, 127]) * float(s[0]), rtol=0, atol=0)


def test_ties_go_to_even():
    # absmax 127 gives scale exactly 1: 2.5 -> 2, 3.5 -> 4, -0.5 -> 0, -1.5 -> -2
    x = np.array([[127.0, 2.5, 3.5, -0.5, -1.5, 0.0]], np.float16)
    c, s = oracle.int8_quantize(x)
    assert s[0] == 1.0
    assert c.tolist() == [[127, 2, 4, 0, -2, 0]]


def test_zero_row_and_absmax_element():
    c, s = oracle.int8_quantize(np.zeros((2, 8), np.float16))
    assert np.all(c == 0) and np.all(s == 0)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, 128)).astype(np.float16)
    c, s = oracle.int8_quantize(x)
    j = np.argmax(np.abs(x.astype(np.float32)), axis=-1)
    # the largest element maps to +-127 with its own sign
    got = c[np.arange(500), j].astype(int)
    assert np.all(np.abs(got) == 127)
    assert np.all(np.sign(got) == np.sign(x[np.arange(500), j].astype(np.float32)))
    assert c.min() >= -127 and c.max() <= 127


def test_round_trip_error_is_half_a_step():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((300, 64)) * np.exp(rng.standard_normal((300, 1)))).astype(np.float16)
    c, s = oracle.int8_quantize(x)
    err = np.abs(oracle.int8_dequantize(c, s) - x.astype(np.float64))
    # rounding to the nearest code: at most half a step, plus the float32
    # rounding of the division (about 127 ulps of a step at most)
    assert np.all(err <= (0.5 + 1e-4) * s[:, None].astype(np.float64) + 1e-12)


def test_storage_ratio():
    # ~2x: d + 4 bytes against 2 d of fp16 (page 3's "~2x")
    assert oracle.int8_bytes_per_token_head(128) == 132
    assert 1.9 < 256 / 132 < 2.0


def test_codes_equal_the_exact_rational_definition():
    # brute force: every code against round(127 x / max|x|) computed in
    # exact rationals, on rows that mix ordinary values with exact halves of
    # the code grid (127 x / a = k + 1/2) and subnormal fp16 values
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((60, 16)) * np.exp(2 * rng.standard_normal((60, 1)))).astype(np.float16)
    x[::3, 0] = np.float16(127.0)
    x[::3, 1:6] = (rng.integers(-127, 127, (20, 5)) + 0.5).astype(np.float16)   # exact ties
    x[1::3, 2] = np.float16(6e-8)
    c, s = oracle.int8_quantize(x)
    for i in range(x.shape[0]):
        a = max(abs(float(e)) for e in x[i])
        for j in range(x.shape[1]):
            assert int(c[i, j]) == _exact_code(x[i, j], a), (i, j)
        assert s[i] == np.float32(Fraction(a) / 127)


def test_float32_route_is_not_the_definition():
    # a row whose element 3 sits exactly on a half step: 127 * 51.625 /
    # 103.25 = 63.5, which the definition rounds to the even 64; dividing by
    # the float32 scale a / 127 instead gives 63.499996 and so 63.  The oracle
    # keeps the definition.
    x = np.array([[-34.6, 53.6, 39.16, 51.62, 23.88, -64.8, 92.9, -103.25]], np.float16)
    assert float(x[0, 3]) == 51.625 and float(x[0, 7]) == -103.25
    assert oracle.int8_levels(x)[0, 3] == 63.5
    c, s = oracle.int8_quantize(x)
    assert int(c[0, 3]) == 64
    v32 = np.float32(x[0, 3]) / np.float32(np.float32(103.25) / np.float32(127.0))
    assert np.rint(v32) == 63

"""Pins of the oracle's INT8 per-token absmax codec (mlxcel "TurboQuant KV
cache", "Available modes": int8, per-token INT8 absmax, about 2x)."""
import numpy as np
import pytest

import oracle


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

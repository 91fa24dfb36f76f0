"""Pins for the oracle's quantize / pack / dequantize steps.

Checked against: brute-force nearest centroid (with constructed ties), packed
words derived by hand and by big-integer arithmetic from the layout
definition, the exact expected distortion for Gaussian inputs (a uniformly
random direction, whatever the rotation), idempotence of quantize after
dequantize, and the zero-vector case.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import read_golden


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4), (32, 1), (128, 2), (64, 5)])
def test_threshold_count_is_nearest_centroid(d, bits):
    c, t = oracle.lloyd_max(d, bits)
    rng = np.random.default_rng(bits * 1000 + d)
    y = rng.uniform(-1.5, 1.5, 200000) * (c[-1] * 1.3)
    brute = np.argmin(np.abs(y[:, None] - c[None, :]), axis=1)  # first index on ties
    assert np.array_equal(oracle.codes_from_rotated(y, t), brute)
    # exact ties: y on a threshold takes the lower code
    assert np.array_equal(oracle.codes_from_rotated(t, t), np.arange(len(t)))
    # just above a threshold takes the upper code
    assert np.array_equal(oracle.codes_from_rotated(np.nextafter(t, np.inf), t), np.arange(1, len(t) + 1))


def _bigint_pack(codes, bits):
    v = 0
    for j, c in enumerate(codes):
        v |= int(c) << (bits * j)
    W = (bits * len(codes) + 31) // 32
    return [(v >> (32 * w)) & 0xFFFFFFFF for w in range(W)]


def test_pack_golden_words():
    for row in read_golden("packing.txt"):
        f = row.split()
        bits, d, pattern = int(f[0]), int(f[1]), f[2]
        want = [int(x, 16) for x in f[3:]]
        codes = (np.arange(d) % (1 << bits)) if pattern == "mod" else np.full(d, (1 << bits) - 1)
        got = oracle.pack_codes(codes[None, :], bits)[0]
        assert [int(x) for x in got] == want
        assert np.array_equal(oracle.unpack_codes(got[None], bits, d)[0], codes)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_pack_roundtrip_and_bigint(bits, d):
    rng = np.random.default_rng(bits * 7 + d)
    codes = rng.integers(0, 1 << bits, size=(5, d))
    words = oracle.pack_codes(codes, bits)
    assert words.dtype == np.uint32
    assert words.shape == (5, oracle.row_words(d, bits))
    assert np.array_equal(oracle.unpack_codes(words, bits, d), codes)
    for r in range(5):
        assert [int(x) for x in words[r]] == _bigint_pack(codes[r], bits)
    # all codes at their maximum sets every bit of the row
    full = oracle.pack_codes(np.full((1, d), (1 << bits) - 1), bits)
    assert np.all(full == 0xFFFFFFFF)


def test_pack_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.array([[16, 0]]), 4)


@pytest.mark.parametrize("d,bits", [(64, 3), (64, 4), (128, 3), (128, 4)])
def test_distortion_on_gaussian_rows(d, bits):
    """For i.i.d. Gaussian rows u = x/|x| is uniform on the sphere, so y = R u
    is uniform too and E|u - u~|^2 = d * D_b(d) exactly; the empirical mean
    over many rows must sit within 4 standard errors."""
    rng = np.random.default_rng(99 + d + bits)
    x = rng.standard_normal((40000, d))
    R = oracle.rotation_matrix(0, d)
    c, t = oracle.lloyd_max(d, bits)
    codes, n, y = oracle.quantize(x, R, t)
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    ut = oracle.dequantize(codes, np.ones(len(x)), R, c)
    err = np.sum((u - ut) ** 2, axis=1)
    want = d * oracle.distortion(d, c, t)
    se = err.std() / math.sqrt(len(err))
    assert abs(err.mean() - want) < 4 * se, (err.mean(), want, se)


def test_quantize_norms_and_rotated_coordinates():
    k, _ = synth.kv_numpy(1, 1, 2, 16, 64)
    R = oracle.rotation_matrix(0, 64)
    _, t = oracle.lloyd_max(64, 3)
    codes, n, y = oracle.quantize(k, R, t)
    xf = k.astype(np.float64)
    assert np.allclose(n, np.linalg.norm(xf, axis=-1), rtol=1e-15)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    assert codes.shape == k.shape and codes.min() >= 0 and codes.max() < 8


@pytest.mark.parametrize("d,bits", [(64, 3), (128, 4)])
def test_requantize_is_idempotent(d, bits):
    k, _ = synth.kv_numpy(3, 1, 2, 200, d, dist="channel", outlier_frac=0.01)
    R = oracle.rotation_matrix(0, d)
    c, t = oracle.lloyd_max(d, bits)
    codes, n, _ = oracle.quantize(k, R, t)
    xt = oracle.dequantize(codes, n, R, c)
    codes2, n2, y2 = oracle.quantize(xt.astype(np.float64), R, t)
    near = np.min(np.abs(y2[..., None] - t), axis=-1) < 1e-9
    assert np.all((codes2 == codes) | near)
    assert np.mean(codes2 == codes) > 0.999


def test_zero_row():
    R = oracle.rotation_matrix(0, 64)
    c, t = oracle.lloyd_max(64, 4)
    codes, n, y = oracle.quantize(np.zeros((1, 64), np.float16), R, t)
    assert n[0] == 0.0
    assert np.all(codes == 7)
    assert np.all(oracle.dequantize(codes, n, R, c) == 0.0)


def test_dequantize_is_inverse_rotation_of_centroids():
    d, bits = 32, 2
    R = oracle.rotation_matrix(5, d)
    c, t = oracle.lloyd_max(d, bits)
    codes = np.arange(d) % 4
    xt = oracle.dequantize(codes[None], np.array([2.0]), R, c)[0]
    assert np.allclose(R @ xt, 2.0 * c[codes], atol=1e-15)

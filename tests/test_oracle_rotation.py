"""Pins for the oracle's rotation (seeded sign-diagonal Walsh-Hadamard).

Checked against: the published SplitMix64 test vector, the Kronecker
definition of the Sylvester matrix, an independent butterfly FWHT, and the
exact integer identities H H^T = d I and H (H x) = d x.
"""
import numpy as np
import pytest

import oracle
from conftest import read_golden


def test_splitmix64_published_vector():
    want = [int(x, 16) for x in read_golden("splitmix64_seed0.txt")]
    assert oracle.splitmix64(0, 3) == want


def test_sign_vector_from_top_bits():
    # 0xe2... has its top bit set, 0x6e... and 0x06... do not.
    assert list(oracle.sign_vector(0, 3)) == [-1.0, 1.0, 1.0]
    s = oracle.sign_vector(12345, 256)
    assert set(np.unique(s)) <= {-1.0, 1.0}
    # a different seed gives a different pattern
    assert np.any(s != oracle.sign_vector(12346, 256))


def _kron_hadamard(d):
    h = np.array([[1]], dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def _butterfly_fwht(x):
    """In-place butterflies, stride 1, 2, 4, ...: (a, b) -> (a + b, a - b)."""
    x = np.array(x, dtype=np.int64, copy=True)
    d = x.shape[-1]
    h = 1
    while h < d:
        for i in range(0, d, 2 * h):
            a = x[..., i:i + h].copy()
            b = x[..., i + h:i + 2 * h].copy()
            x[..., i:i + h] = a + b
            x[..., i + h:i + 2 * h] = a - b
        h *= 2
    return x


@pytest.mark.parametrize("d", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_sylvester_equals_kronecker(d):
    assert np.array_equal(oracle.sylvester_hadamard(d), _kron_hadamard(d))


@pytest.mark.parametrize("d", [2, 8, 32, 64, 128, 256])
def test_hadamard_integer_identities(d):
    H = oracle.sylvester_hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d, dtype=np.int64))
    rng = np.random.default_rng(d)
    x = rng.integers(-1000, 1000, size=(7, d))
    assert np.array_equal((x @ H.T) @ H.T, d * x)


@pytest.mark.parametrize("d", [2, 4, 16, 64, 128, 256])
def test_butterfly_fwht_equals_matrix(d):
    H = oracle.sylvester_hadamard(d)
    rng = np.random.default_rng(7 + d)
    x = rng.integers(-50, 50, size=(5, d))
    assert np.array_equal(_butterfly_fwht(x), x @ H.T)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_rotation_orthonormal(d):
    R = oracle.rotation_matrix(0, d)
    assert np.max(np.abs(R.T @ R - np.eye(d))) < 1e-14
    rng = np.random.default_rng(d)
    x = rng.standard_normal((4, d))
    assert np.allclose(np.linalg.norm(x @ R.T, axis=1), np.linalg.norm(x, axis=1), rtol=1e-15, atol=0)
    assert np.max(np.abs((x @ R.T) @ R - x)) < 1e-14
    # signs are applied before H: R = H diag(s) / sqrt(d)
    s = oracle.sign_vector(0, d)
    e0 = np.zeros(d); e0[0] = 1.0
    assert np.allclose(R @ e0, s[0] * oracle.sylvester_hadamard(d)[:, 0] / np.sqrt(d))


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        oracle.sylvester_hadamard(80)

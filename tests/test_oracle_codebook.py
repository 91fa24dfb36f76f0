"""Pins for the oracle's coordinate pdf and Lloyd-Max codebook.

Checked against: numerical quadrature of the pdf (normalisation, E[X^2] =
1/d, tails and moments), the 1-bit closed form, the Lloyd-Max fixed-point
conditions recomputed by Gauss-Legendre quadrature, an unconstrained
(both-halves) Lloyd iteration from a different start, and the Gaussian
Lloyd-Max limits of Max (1960) as d grows.
"""
import math

import numpy as np
import pytest
from scipy import integrate
from scipy.special import gammaln
from scipy.stats import norm

import oracle
from conftest import read_golden


def _quad(f, a, b):
    return integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-13, limit=200)[0]


@pytest.mark.parametrize("d", [3, 4, 16, 64, 128])
def test_pdf_normalised_and_second_moment(d):
    f = lambda x: float(oracle.coord_pdf(x, d))
    assert abs(_quad(f, -1, 1) - 1.0) < 1e-12
    assert abs(_quad(lambda x: x * x * f(x), -1, 1) - 1.0 / d) < 1e-12


@pytest.mark.parametrize("d", [8, 64, 128])
def test_cell_integrals_match_quadrature(d):
    f = lambda x: float(oracle.coord_pdf(x, d))
    for lo, hi in [(-0.3, -0.1), (-0.05, 0.2), (0.1, 0.45), (0.0, 1.0)]:
        assert abs(float(oracle.cell_mass(lo, hi, d)) - _quad(f, lo, hi)) < 1e-12
        assert abs(float(oracle.cell_first_moment(lo, hi, d)) - _quad(lambda x: x * f(x), lo, hi)) < 1e-12
        assert abs(float(oracle.cell_second_moment(lo, hi, d)) - _quad(lambda x: x * x * f(x), lo, hi)) < 1e-12
    for t in [-0.5, -0.1, 0.0, 0.07, 0.3]:
        assert abs(float(oracle.coord_tail(t, d)) - _quad(f, t, 1)) < 1e-12


@pytest.mark.parametrize("d", [16, 64, 128, 1024])
def test_one_bit_closed_form(d):
    c, t = oracle.lloyd_max(d, 1)
    want = math.exp(gammaln(d / 2) - gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert np.allclose(c, [-want, want], rtol=0, atol=1e-13)
    assert t[0] == 0.0
    assert abs(oracle.distortion(d, c, t) - (1.0 / d - want * want)) < 1e-13


def _gl_cell(f, lo, hi, n=64):
    x, w = np.polynomial.legendre.leggauss(n)
    xm = 0.5 * (hi - lo) * x + 0.5 * (hi + lo)
    return 0.5 * (hi - lo) * np.sum(w * f(xm))


@pytest.mark.parametrize("d", [32, 64, 128, 256])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_fixed_point_conditions(d, bits):
    c, t = oracle.lloyd_max(d, bits)
    L = 1 << bits
    assert c.shape == (L,) and t.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    # antisymmetric codebook, middle threshold exactly 0, midpoints
    assert np.array_equal(c, -c[::-1])
    assert t[L // 2 - 1] == 0.0
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-16
    # each centroid is the conditional mean of its cell (independent
    # Gauss-Legendre quadrature of the unnormalised density)
    g = lambda x: (1.0 - x * x) ** ((d - 3) / 2.0)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(L):
        lo, hi = edges[k], edges[k + 1]
        m0 = sum(_gl_cell(g, a, b) for a, b in zip(np.linspace(lo, hi, 9)[:-1], np.linspace(lo, hi, 9)[1:]))
        m1 = sum(_gl_cell(lambda x: x * g(x), a, b) for a, b in zip(np.linspace(lo, hi, 9)[:-1], np.linspace(lo, hi, 9)[1:]))
        assert abs(m1 / m0 - c[k]) < 1e-12, (k, m1 / m0, c[k])


@pytest.mark.parametrize("d,bits", [(64, 2), (128, 3), (32, 3)])
def test_unconstrained_lloyd_from_other_start(d, bits):
    """Full (both halves) Lloyd iteration, uniform start, own quadrature:
    converges to the oracle's codebook (unique fixed point, log-concave pdf)."""
    L = 1 << bits
    g = lambda x: (1.0 - x * x) ** ((d - 3) / 2.0)
    c = np.linspace(-2.0, 2.0, L) / math.sqrt(d)
    for _ in range(3000):
        e = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        new = np.array([
            sum(_gl_cell(lambda x: x * g(x), a, b, 24) for a, b in zip(np.linspace(e[k], e[k + 1], 5)[:-1], np.linspace(e[k], e[k + 1], 5)[1:]))
            / sum(_gl_cell(g, a, b, 24) for a, b in zip(np.linspace(e[k], e[k + 1], 5)[:-1], np.linspace(e[k], e[k + 1], 5)[1:]))
            for k in range(L)])
        done = np.max(np.abs(new - c)) < 1e-15
        c = new
        if done:
            break
    want, _ = oracle.lloyd_max(d, bits)
    assert np.max(np.abs(c - want)) < 1e-12


def _gaussian_lloyd_max(bits, iters=20000):
    """Lloyd-Max for N(0, 1) with closed-form conditional means
    (phi(a) - phi(b)) / (Phi(b) - Phi(a)).  Returns (centroids, mse)."""
    L = 1 << bits
    c = norm.ppf((np.arange(L) + 0.5) / L)
    for _ in range(iters):
        e = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        p = norm.cdf(e[1:]) - norm.cdf(e[:-1])
        new = (norm.pdf(e[:-1]) - norm.pdf(e[1:])) / p
        if np.max(np.abs(new - c)) < 1e-15:
            c = new
            break
        c = new
    e = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
    p = norm.cdf(e[1:]) - norm.cdf(e[:-1])
    return c, 1.0 - float(np.sum(c * c * p))


def test_gaussian_reference_matches_max_table():
    for row in read_golden("gaussian_lloyd_max.txt"):
        bits, mse = row.split()
        _, got = _gaussian_lloyd_max(int(bits))
        assert abs(got - float(mse)) / float(mse) < 5e-4, (bits, got, mse)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_limit(bits):
    """d * D_b(d) and sqrt(d) * c approach the Gaussian Lloyd-Max values, with
    the gap shrinking monotonically in d."""
    cg, mse_g = _gaussian_lloyd_max(bits)
    gaps, cgaps = [], []
    for d in [64, 256, 1024, 4096, 16384, 65536]:
        c, t = oracle.lloyd_max(d, bits)
        gaps.append(abs(d * oracle.distortion(d, c, t) - mse_g))
        cgaps.append(np.max(np.abs(math.sqrt(d) * c - cg)))
    assert all(a > b for a, b in zip(gaps, gaps[1:])), gaps
    assert all(a > b for a, b in zip(cgaps, cgaps[1:])), cgaps
    assert gaps[-1] / mse_g < 1e-3
    assert cgaps[-1] < 1e-3


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_identity_at_fixed_point(d, bits):
    """At the fixed point D = E[X^2] - sum_k c_k^2 P_k."""
    c, t = oracle.lloyd_max(d, bits)
    e = np.concatenate(([-1.0], t, [1.0]))
    P = oracle.cell_mass(e[:-1], e[1:], d)
    assert abs(oracle.distortion(d, c, t) - (1.0 / d - np.sum(c * c * P))) < 1e-14

"""Pins for the oracle's Lloyd-Max codebooks (CPU only).

Each check compares the oracle with something other than itself: values printed on
the pages, a closed form, an independent library quadrature, the Gaussian limit,
or a Monte-Carlo estimate.
"""

import json
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codebook as cbm

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_symmetry_and_middle_boundary(bits):
    b, c = cbm.codebook(bits)
    L = 1 << bits
    assert b.shape == (L - 1,) and c.shape == (L,)
    assert b[L // 2 - 1] == 0.0
    np.testing.assert_array_equal(c, -c[::-1])
    np.testing.assert_array_equal(b, -b[::-1])
    assert np.all(np.diff(b) > 0) and np.all(np.diff(c) > 0)
    # each boundary lies between its neighbouring centroids
    assert np.all(c[:-1] < b) and np.all(b < c[1:])


def test_turboq2_printed_centroids():
    """[turboq] 'Encode pipeline' prints the 2-bit d=128 centroids {+-0.040, +-0.133}."""
    g = GOLDEN["turboq2_centroids_d128"]
    _, c = cbm.codebook(2, 128)
    np.testing.assert_array_equal(np.round(c.astype(np.float64), g["decimals"]), g["values"])


def test_one_bit_closed_form():
    """1 level pair: the centroid is E[y | y > 0] = 1 / ((m+1) B(1/2, m+1))."""
    for dim in (64, 128, 256):
        m = cbm.m_beta(dim)
        _, c, _ = cbm.lloyd_max_fp64(1, dim)
        expect = 1.0 / ((m + 1.0) * special.beta(0.5, m + 1.0))
        assert abs(c[1] - expect) < 1e-13 * expect


def test_distortion_monotone_in_bits():
    m = cbm.m_beta(128)
    D = [cbm.distortion(*cbm.lloyd_max_fp64(b)[:2], m) for b in (1, 2, 3, 4)]
    assert D[0] > D[1] > D[2] > D[3] > 0


def _gauss_lloyd(bits, iters=5000):
    """Gaussian N(0,1) Lloyd-Max by the textbook closed forms (scipy.stats.norm)."""
    L = 1 << bits
    b = np.linspace(-2.0, 2.0, L + 1)[1:-1]
    for _ in range(iters):
        e = np.concatenate(([-np.inf], b, [np.inf]))
        c = (stats.norm.pdf(e[:-1]) - stats.norm.pdf(e[1:])) / (
            stats.norm.cdf(e[1:]) - stats.norm.cdf(e[:-1]))
        b = 0.5 * (c[:-1] + c[1:])
    return b, c


@pytest.mark.parametrize("bits", [2, 3])
def test_gaussian_limit(bits):
    """For large d, (1 - y^2)^m -> exp(-m y^2): sqrt(2m) * levels -> N(0,1) Lloyd-Max."""
    dim = 1 << 15
    m = cbm.m_beta(dim)
    gb, gc = _gauss_lloyd(bits)
    # the uniform start has cells of zero fp64 mass at this d; start instead from a
    # guess 10 % off the scaled Gaussian levels (the fixed point is unique)
    init = 1.1 * gb[len(gb) // 2 + 1:] / np.sqrt(2 * m)
    b, c, _ = cbm.lloyd_max_fp64(bits, dim, tol=1e-13, init=init)
    np.testing.assert_allclose(np.sqrt(2 * m) * c, gc, rtol=2e-3, atol=2e-3)
    np.testing.assert_allclose(np.sqrt(2 * m) * b, gb, rtol=2e-3, atol=2e-3)


def _quad_distortion(b, c, m):
    """E (y - Q(y))^2 by scipy.integrate.quad, cell by cell (independent quadrature)."""
    f = lambda y: (1.0 - y * y) ** m  # noqa: E731
    edges = np.concatenate(([-1.0], b, [1.0]))
    num = sum(integrate.quad(lambda y, cj=cj: (y - cj) ** 2 * f(y), lo, hi,
                             epsabs=0, epsrel=1e-12, limit=200)[0]
              for lo, hi, cj in zip(edges[:-1], edges[1:], c))
    den = integrate.quad(f, -1.0, 1.0, epsabs=0, epsrel=1e-13, limit=200)[0]
    return num / den


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_distortion_matches_independent_quadrature(bits):
    m = cbm.m_beta(128)
    b, c, _ = cbm.lloyd_max_fp64(bits)
    assert abs(cbm.distortion(b, c, m) - _quad_distortion(b, c, m)) < 1e-9 * cbm.distortion(b, c, m)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_local_optimality(bits):
    """Moving any centroid or boundary off the fixed point raises the distortion."""
    m = cbm.m_beta(128)
    b, c, _ = cbm.lloyd_max_fp64(bits)
    d0 = _quad_distortion(b, c, m)
    for i in range(len(c)):
        for eps in (-1e-3, 1e-3):
            cc = c.copy()
            cc[i] += eps
            assert _quad_distortion(b, cc, m) > d0
    for i in range(len(b)):
        for eps in (-1e-3, 1e-3):
            bb = b.copy()
            bb[i] += eps
            if np.all(np.diff(bb) > 0):
                assert _quad_distortion(bb, c, m) > d0


@pytest.mark.parametrize("bits", [2, 4])
def test_fixed_point_independent_of_start(bits):
    """Lloyd-Max is unique for this log-concave density: any start converges to it."""
    rng = np.random.default_rng(5)
    L = 1 << bits
    init = np.sort(rng.uniform(0.01, 0.9, size=L // 2 - 1))
    b0, c0, _ = cbm.lloyd_max_fp64(bits)
    b1, c1, _ = cbm.lloyd_max_fp64(bits, init=init)
    np.testing.assert_allclose(c1, c0, rtol=0, atol=1e-10)
    assert np.array_equal(c1.astype(np.float32), c0.astype(np.float32))


def test_distortion_monte_carlo_on_sphere():
    """MSE of the quantizer on coordinates of uniform unit vectors equals the
    distortion under the exact sphere marginal (m' = (d-3)/2)."""
    rng = np.random.default_rng(11)
    g = rng.standard_normal((20000, 128))
    u = g / np.linalg.norm(g, axis=1, keepdims=True)
    for bits in (2, 4):
        b, c = cbm.codebook(bits)
        q = c[np.searchsorted(b, u.astype(np.float32), side="left")].astype(np.float64)
        mse = np.mean((u - q) ** 2)
        expect = cbm.distortion(b, c, cbm.m_sphere(128))
        assert abs(mse - expect) < 0.01 * expect

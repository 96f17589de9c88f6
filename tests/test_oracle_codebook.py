"""Pins of the oracle's Lloyd-Max codebook against things other than itself:
the sphere-coordinate law by Monte Carlo, adaptive quadrature, the textbook
1-bit closed form, Max's Gaussian table in the large-d limit, and uniqueness."""
import json
import os

import numpy as np
import pytest
from scipy import integrate, stats
from scipy.special import gammaln

from oracle import codebook as cbm


@pytest.mark.parametrize("d", [5, 16, 128])
def test_density_is_the_sphere_coordinate_law(d):
    # a uniform point on S^{d-1} is a normalised Gaussian vector; its first
    # coordinate must follow coord_cdf (Kolmogorov-Smirnov, large sample)
    rng = np.random.default_rng(1234 + d)
    g = rng.standard_normal((200000, d))
    x = g[:, 0] / np.linalg.norm(g, axis=1)
    res = stats.kstest(x, lambda t: cbm.coord_cdf(t, d))
    assert res.pvalue > 1e-3
    # and the density integrates to one and is the derivative of the cdf
    mass, _ = integrate.quad(lambda t: cbm.coord_density(t, d), -1, 1, epsabs=1e-13)
    assert abs(mass - 1) < 1e-10
    for t in (-0.3, 0.01, 0.2):
        h = 1e-6
        num = (cbm.coord_cdf(t + h, d) - cbm.coord_cdf(t - h, d)) / (2 * h)
        assert abs(num - cbm.coord_density(t, d)) < 1e-6 * max(1, cbm.coord_density(t, d))


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_conditions(bits):
    d = 128
    cb = cbm.lloyd_max(d, bits)
    c, t = cb.centroids, cb.thresholds
    assert c.shape == (1 << bits,) and t.shape == ((1 << bits) - 1,)
    assert np.all(np.diff(c) > 0)
    # midpoint condition
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-15
    # centroid condition, checked with independent adaptive quadrature
    edges = cb.boundaries
    f = lambda x: cbm.coord_density(x, d)  # noqa: E731
    for k in range(len(c)):
        lo, hi = edges[k], edges[k + 1]
        m0, _ = integrate.quad(f, lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)
        m1, _ = integrate.quad(lambda x: x * f(x), lo, hi, epsabs=1e-15, epsrel=1e-13, limit=200)
        assert abs(m1 / m0 - c[k]) < 1e-12
    # symmetry of the optimum for a symmetric law
    assert np.max(np.abs(c + c[::-1])) < 1e-14


def test_one_bit_closed_form():
    # 1 bit: the cells are the half-lines, the centroids are +-E|X| =
    # +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); 0.0706616 at d = 128
    for d in (16, 128, 1000):
        cb = cbm.lloyd_max(d, 1)
        ref = np.exp(gammaln(d / 2) - 0.5 * np.log(np.pi) - gammaln((d + 1) / 2))
        assert abs(cb.centroids[1] - ref) < 1e-12 * ref
        assert abs(cb.thresholds[0]) < 1e-15
    assert abs(cbm.lloyd_max(128, 1).centroids[1] - 0.0706616) < 1e-7


def test_large_d_tends_to_max_gaussian_table(golden_dir):
    gold = json.load(open(os.path.join(golden_dir, "gaussian_lloyd_max.json")))
    d = 10000
    for bits_s, pos in gold["levels"].items():
        bits = int(bits_s)
        cb = cbm.lloyd_max(d, bits, tol=1e-12 / np.sqrt(d))
        got = np.sqrt(d) * cb.centroids[1 << (bits - 1):]
        # O(1/d) finite-d offset plus the table's 4-digit rounding
        assert np.max(np.abs(got - np.array(pos))) < 5e-4, (bits, got, pos)


def test_fixed_point_is_unique():
    ref = cbm.lloyd_max(128, 3).centroids
    rng = np.random.default_rng(7)
    for _ in range(3):
        init = np.sort(rng.uniform(-0.5, 0.5, size=8))
        got = cbm.lloyd_max(128, 3, init=init).centroids
        assert np.max(np.abs(got - ref)) < 1e-13


def test_codebook_is_locally_mse_optimal():
    # moving any threshold or centroid off the optimum can only raise the MSE
    d, bits = 128, 2
    cb = cbm.lloyd_max(d, bits)
    rng = np.random.default_rng(3)
    g = rng.standard_normal((400000, d))
    x = g[:, 0] / np.linalg.norm(g, axis=1)

    def mse(c, t):
        idx = np.searchsorted(t, x, side="left")
        return np.mean((x - c[idx]) ** 2)

    base = mse(cb.centroids, cb.thresholds)
    for k in range(len(cb.centroids)):
        for eps in (-3e-3, 3e-3):
            c = cb.centroids.copy()
            c[k] += eps
            assert mse(c, cb.thresholds) > base

"""Pins for the oracle's magnitude codebook (the Beta-prior Lloyd-Max quantiser).

The oracle derives the codebook through the regularised incomplete beta
function.  These checks use other routes: direct numerical quadrature of the
density of one coordinate of a uniform unit vector, and Monte-Carlo sampling
of such vectors.
"""
import math
import warnings

import numpy as np
from scipy import integrate, special

warnings.filterwarnings("ignore", category=integrate.IntegrationWarning)

from oracle.codebook import bin_mass, lloyd_max, spec_tables

M = 8


def density(a, m=M):
    """Density of |u_j| for u uniform on the unit sphere of R^m:
    proportional to (1 - a^2)^((m-3)/2) on [0, 1]."""
    return (1 - a * a) ** ((m - 3) / 2) / special.beta(0.5, (m - 1) / 2) * 2


def test_density_normalised():
    val, _ = integrate.quad(density, 0, 1, epsabs=1e-14, epsrel=1e-14)
    assert abs(val - 1) < 1e-12


def check_lloyd_max_conditions(levels, thresholds):
    """Every level is the conditional mean of its bin (quadrature) and every
    threshold the midpoint of its neighbours."""
    edges = np.concatenate([[0.0], thresholds, [1.0]])
    for i, c in enumerate(levels):
        num, _ = integrate.quad(lambda a: a * density(a), edges[i], edges[i + 1],
                                epsabs=1e-15, epsrel=1e-14)
        den, _ = integrate.quad(density, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-14)
        if abs(num / den - c) > 1e-12:
            return False
    return np.allclose(thresholds, 0.5 * (levels[:-1] + levels[1:]), atol=1e-13, rtol=0)


def test_lloyd_max_conditions():
    c, t = lloyd_max(M)
    assert np.all(np.diff(c) > 0) and 0 < c[0] and c[-1] < 1
    assert check_lloyd_max_conditions(c, t)


def test_lloyd_max_is_a_local_mse_minimum():
    c, t = lloyd_max(M)

    def mse(levels):
        th = 0.5 * (levels[:-1] + levels[1:])
        edges = np.concatenate([[0.0], th, [1.0]])
        return sum(integrate.quad(lambda a: (a - levels[i]) ** 2 * density(a),
                                  edges[i], edges[i + 1], epsabs=1e-15)[0]
                   for i in range(len(levels)))
    base = mse(c)
    rng = np.random.default_rng(0)
    for _ in range(10):
        assert mse(c + rng.normal(0, 2e-3, c.shape)) > base
    assert 5e-4 < base < 2e-3


def test_bin_masses_against_monte_carlo():
    """Bin probabilities of |u_j| for uniform directions in R^8."""
    c, t = lloyd_max(M)
    rng = np.random.default_rng(1)
    z = rng.standard_normal((400_000, M))
    u = np.abs(z / np.linalg.norm(z, axis=1, keepdims=True)).ravel()
    counts = np.bincount(np.searchsorted(t, u, side="right"), minlength=8)
    n = u.size
    edges = np.concatenate([[0.0], t, [1.0]])
    for i in range(8):
        p = bin_mass(edges[i], edges[i + 1], M)
        sd = math.sqrt(p * (1 - p) / n) * math.sqrt(M)   # coordinates of one vector correlate
        assert abs(counts[i] / n - p) < 5 * sd
    assert abs(sum(bin_mass(edges[i], edges[i + 1], M) for i in range(8)) - 1) < 1e-14


def test_spec_tables_are_rounded_once():
    c, t = lloyd_max(M)
    c32, T32 = spec_tables(M)
    assert c32.dtype == np.float32 and T32.dtype == np.float32
    assert np.array_equal(c32, c.astype(np.float32))
    assert np.array_equal(T32, (t * t).astype(np.float32))
    assert np.all(np.diff(T32) > 0)


# ----------------------------------------------------------- quantile reading

def check_quantile_conditions(levels, thresholds):
    """Equal-probability bins (each 1/8 of the mass, by quadrature of the density)
    and every level the conditional mean of its bin (quadrature)."""
    edges = np.concatenate([[0.0], thresholds, [1.0]])
    for i, c in enumerate(levels):
        den, _ = integrate.quad(density, edges[i], edges[i + 1], epsabs=1e-15, epsrel=1e-14)
        if abs(den - 1.0 / len(levels)) > 1e-11:
            return False
        num, _ = integrate.quad(lambda a: a * density(a), edges[i], edges[i + 1],
                                epsabs=1e-15, epsrel=1e-14)
        if abs(num / den - c) > 1e-12:
            return False
    return True


def test_quantile_codebook_conditions():
    from oracle.codebook import quantile_codebook
    c, t = quantile_codebook(M)
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    assert np.all((t > c[:-1]) & (t < c[1:]))          # each threshold between its levels
    assert check_quantile_conditions(c, t)


def test_quantile_bins_against_monte_carlo():
    from oracle.codebook import quantile_codebook
    _, t = quantile_codebook(M)
    rng = np.random.default_rng(2)
    z = rng.standard_normal((400_000, M))
    u = np.abs(z / np.linalg.norm(z, axis=1, keepdims=True)).ravel()
    frac = np.bincount(np.searchsorted(t, u, side="right"), minlength=8) / u.size
    sd = math.sqrt(0.125 * 0.875 / u.size) * math.sqrt(M)
    assert np.all(np.abs(frac - 0.125) < 5 * sd)


def test_mutation_quantile_midpoint_thresholds_is_caught():
    """Lloyd-Max thresholds (midpoints) do not give equal bins: the quantile pin
    rejects them."""
    c, t = lloyd_max(M)
    assert not check_quantile_conditions(c, t)

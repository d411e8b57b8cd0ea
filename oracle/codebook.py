"""Oracle (test infrastructure): the 3-bit magnitude codebook of the RSQ-IP code.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package; the HIP library never does and computes its own codebook.

ParisKV page, "Candidate reranking (RSQ-IP) > Quantization": every coordinate of
a rotated, normalised subspace direction is coded with one sign bit and a
3-bit magnitude whose codebook comes from the Beta prior that the random
rotation induces.

Reading used here: for a direction u drawn uniformly from the unit sphere in
R^m (what a random rotation makes of any fixed direction), every squared
coordinate u_j^2 follows Beta(1/2, (m-1)/2).  The 8 magnitude levels are the
Lloyd-Max (minimum mean-squared error) quantiser of |u_j| under that law:
each level is the conditional mean of its bin and each threshold is the
midpoint of its two neighbouring levels.

Everything here is float64 and uses only the regularised incomplete beta
function (scipy.special.betainc) and its inverse.
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _beta_params(m: int):
    return 0.5, (m - 1) / 2.0


def bin_mass(lo: float, hi: float, m: int) -> float:
    """P(lo <= |u_j| < hi) for u uniform on the unit sphere of R^m."""
    a, b = _beta_params(m)
    return float(special.betainc(a, b, hi * hi) - special.betainc(a, b, lo * lo))


def bin_first_moment(lo: float, hi: float, m: int) -> float:
    """E[|u_j| ; lo <= |u_j| < hi].

    With X = u_j^2 ~ Beta(a, b): E[sqrt(X) 1{X in I}] = B(a+1/2, b)/B(a, b) *
    P(X' in I) where X' ~ Beta(a+1/2, b).
    """
    a, b = _beta_params(m)
    ratio = np.exp(special.betaln(a + 0.5, b) - special.betaln(a, b))
    return float(ratio * (special.betainc(a + 0.5, b, hi * hi) -
                          special.betainc(a + 0.5, b, lo * lo)))


def lloyd_max(m: int = 8, n_levels: int = 8, tol: float = 1e-15, max_iter: int = 100000):
    """Lloyd-Max levels c[0..n-1] and thresholds t[1..n-1] (as t[0..n-2]) for |u_j|.

    Starts from equal-probability bins and alternates the two optimality
    conditions until the thresholds stop moving.
    """
    a, b = _beta_params(m)
    q = np.arange(1, n_levels) / n_levels
    t = np.sqrt(special.betaincinv(a, b, q))
    for _ in range(max_iter):
        edges = np.concatenate([[0.0], t, [1.0]])
        c = np.array([bin_first_moment(edges[i], edges[i + 1], m) /
                      bin_mass(edges[i], edges[i + 1], m) for i in range(n_levels)])
        t_new = 0.5 * (c[:-1] + c[1:])
        if np.max(np.abs(t_new - t)) < tol:
            t = t_new
            break
        t = t_new
    edges = np.concatenate([[0.0], t, [1.0]])
    c = np.array([bin_first_moment(edges[i], edges[i + 1], m) /
                  bin_mass(edges[i], edges[i + 1], m) for i in range(n_levels)])
    return c, t


def quantile_codebook(m: int = 8, n_levels: int = 8):
    """The alternative reading of the Beta-prior codebook: equal-probability bins
    (threshold t_l is the l/n quantile of |u_j|) with each level the conditional
    mean of its bin.  Returns (levels c[0..n-1], thresholds t[0..n-2])."""
    a, b = _beta_params(m)
    t = np.sqrt(special.betaincinv(a, b, np.arange(1, n_levels) / n_levels))
    edges = np.concatenate([[0.0], t, [1.0]])
    c = np.array([bin_first_moment(edges[i], edges[i + 1], m) /
                  bin_mass(edges[i], edges[i + 1], m) for i in range(n_levels)])
    return c, t


def spec_tables(m: int = 8, n_levels: int = 8, kind: str = "lloyd_max"):
    """The two fp32 tables the coding rule uses: levels fp32(c_i) and squared
    thresholds fp32(t_l^2) (t_l^2 formed in float64, then rounded once).
    kind: "lloyd_max" (the default reading) or "quantile"."""
    c, t = (lloyd_max if kind == "lloyd_max" else quantile_codebook)(m, n_levels)
    return c.astype(np.float32), (t * t).astype(np.float32)

"""Lloyd-Max scalar codebook for one coordinate of a randomly rotated unit vector.

TEST INFRASTRUCTURE (see the package docstring): float64, scipy special
functions, plain Lloyd iteration.

[explainer] "Ý tưởng cốt lõi": after a fixed random rotation, every coordinate
of a unit vector follows the same concentrated Beta-type law, so one
MSE-optimal scalar quantizer serves every coordinate.  [audit] AUDIT 1 names
the tables the quantizer keeps: ``centroids``, ``boundaries`` and
``decision_boundaries``.

Reading taken: the law is the exact marginal of one coordinate of a uniform
point on the sphere S^{d-1},

    f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),  |x| <= 1,

i.e. (x+1)/2 ~ Beta((d-1)/2, (d-1)/2) (not its N(0, 1/d) approximation).
``decision_boundaries`` are the 2^b - 1 interior thresholds, ``boundaries`` the
2^b + 1 cell edges including -1 and +1.
"""
from __future__ import annotations

import dataclasses

import numpy as np
from scipy.special import betainc, betaincc, betaincinv, gammaln


@dataclasses.dataclass(frozen=True)
class Codebook:
    d: int
    bits: int
    centroids: np.ndarray  # (2^b,) ascending
    thresholds: np.ndarray  # (2^b - 1,) interior decision boundaries
    iterations: int

    @property
    def boundaries(self) -> np.ndarray:
        return np.concatenate([[-1.0], self.thresholds, [1.0]])


def _log_norm_const(d: int) -> float:
    return gammaln(d / 2) - 0.5 * np.log(np.pi) - gammaln((d - 1) / 2)


def coord_density(x, d: int):
    """f_d(x): density of one coordinate of a uniform point on S^{d-1}."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(_log_norm_const(d)) * np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2)


def coord_cdf(x, d: int):
    """P(X <= x) via the regularized incomplete beta function."""
    p = (d - 1) / 2
    return betainc(p, p, (np.asarray(x, dtype=np.float64) + 1.0) / 2.0)


def _cell_mass(lo: np.ndarray, hi: np.ndarray, d: int) -> np.ndarray:
    """P(lo < X <= hi).  Cells in the upper half use the complemented function so
    tail masses keep their relative precision."""
    p = (d - 1) / 2
    a, b = (lo + 1.0) / 2.0, (hi + 1.0) / 2.0
    lower = betainc(p, p, b) - betainc(p, p, a)
    upper = betaincc(p, p, a) - betaincc(p, p, b)
    return np.where((lo + hi) > 0, upper, lower)


def _cell_first_moment(lo: np.ndarray, hi: np.ndarray, d: int) -> np.ndarray:
    """Integral of x f_d(x) over (lo, hi]; the antiderivative of
    x (1-x^2)^a is -(1-x^2)^(a+1) / (2(a+1))."""
    a1 = (d - 3) / 2 + 1
    anti = lambda x: -np.clip(1.0 - x * x, 0.0, None) ** a1 / (2.0 * a1)  # noqa: E731
    return np.exp(_log_norm_const(d)) * (anti(hi) - anti(lo))


def lloyd_max(d: int, bits: int, init: np.ndarray | None = None, tol: float = 1e-15,
              max_iter: int = 200000) -> Codebook:
    """MSE-optimal 2^bits-level scalar quantizer for f_d by Lloyd's iteration:
    thresholds at the midpoints of neighbouring centroids, centroids at the
    conditional means of their cells, repeated until no centroid moves by more
    than ``tol``.  f_d is log-concave, so the fixed point is unique whatever the
    (sorted, distinct) start."""
    if d < 3 or bits < 1:
        raise ValueError("need d >= 3 and bits >= 1")
    levels = 1 << bits
    if init is None:
        # start at the quantiles of the cells' mid-probabilities
        p = (d - 1) / 2
        c = 2.0 * betaincinv(p, p, (np.arange(levels) + 0.5) / levels) - 1.0
    else:
        c = np.sort(np.asarray(init, dtype=np.float64))
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[-1.0], t, [1.0]])
        lo, hi = edges[:-1], edges[1:]
        c_new = _cell_first_moment(lo, hi, d) / _cell_mass(lo, hi, d)
        moved = np.max(np.abs(c_new - c))
        c = c_new
        if moved < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return Codebook(d=d, bits=bits, centroids=c, thresholds=t, iterations=it)

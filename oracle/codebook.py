"""Lloyd-Max codebook for one rotated coordinate (oracle; test infrastructure).

[ZB] paragraph 2: after a random rotation each coordinate follows a Beta law
and an optimal scalar quantizer is applied per coordinate. [WD] "1.
PolarQuant": the rotation is a multiplication by a random orthogonal matrix.

Reading (law): a coordinate y of a uniformly random unit vector in R^d has
density f_d(y) = C_d (1 - y^2)^((d-3)/2) on [-1, 1], i.e. (y + 1)/2 follows
Beta((d-1)/2, (d-1)/2), and y^2 follows Beta(1/2, (d-1)/2). The rotation of
a fixed vector by a Haar orthogonal matrix is exactly such a unit vector
(times the norm). "Optimal" is read as minimum mean squared error, whose
quantizer is the Lloyd-Max fixed point (Lloyd 1957 / Max 1960); f_d is
log-concave for d >= 3, so that fixed point is unique (Fleischer 1964).

Everything is float64 and uses scipy's incomplete beta function.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
from scipy.special import betainc, betaincinv, gammaln


def _normaliser(d: int) -> float:
    # C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2))
    return float(np.exp(gammaln(d / 2.0) - gammaln((d - 1) / 2.0) - 0.5 * np.log(np.pi)))


def coordinate_pdf(y, d: int):
    """f_d(y) = C_d (1 - y^2)^((d-3)/2) on [-1, 1], zero outside."""
    y = np.asarray(y, dtype=np.float64)
    inside = np.abs(y) <= 1.0
    base = np.where(inside, 1.0 - y * y, 0.0)
    return np.where(inside, _normaliser(d) * base ** ((d - 3) / 2.0), 0.0)


def coordinate_cdf(y, d: int):
    """F_d(y) = 1/2 + sign(y)/2 * I_{y^2}(1/2, (d-1)/2), clamped to [-1, 1]."""
    y = np.clip(np.asarray(y, dtype=np.float64), -1.0, 1.0)
    return 0.5 + 0.5 * np.sign(y) * betainc(0.5, (d - 1) / 2.0, y * y)


def coordinate_ppf(u, d: int):
    """Inverse of coordinate_cdf for u in (0, 1)."""
    u = np.asarray(u, dtype=np.float64)
    v = 2.0 * u - 1.0
    return np.sign(v) * np.sqrt(betaincinv(0.5, (d - 1) / 2.0, np.abs(v)))


def cell_first_moment(a, b, d: int):
    """Integral of y f_d(y) over [a, b], in closed form:
    C_d / (d - 1) * ((1 - a^2)^((d-1)/2) - (1 - b^2)^((d-1)/2))."""
    a = np.clip(np.asarray(a, dtype=np.float64), -1.0, 1.0)
    b = np.clip(np.asarray(b, dtype=np.float64), -1.0, 1.0)
    e = (d - 1) / 2.0
    # (1 - y^2)^e evaluated as exp(e log1p(-y^2)) to keep relative precision at large d
    with np.errstate(divide="ignore"):
        pa = np.exp(e * np.log1p(-a * a))
        pb = np.exp(e * np.log1p(-b * b))
    return _normaliser(d) / (d - 1) * (pa - pb)


@dataclass
class Codebook:
    d: int
    mse_bits: int
    centroids: np.ndarray      # L = 2^m increasing values
    boundaries: np.ndarray     # L - 1 midpoints between neighbouring centroids
    mse_per_coord: float       # E[(y - Q(y))^2] under f_d
    iterations: int


def lloyd_max(d: int, mse_bits: int, tol: float | None = None,
              max_iter: int = 200_000, init: np.ndarray | None = None) -> Codebook:
    """Lloyd-Max quantizer with 2^mse_bits levels for the density f_d.

    Steps, in the order of the algorithm:
      1. start from the quantiles F^-1((k + 1/2) / L) (or ``init``);
      2. repeat: boundaries = midpoints of neighbouring centroids (with -1
         and 1 at the ends); each centroid = the conditional mean of its
         cell, from the closed-form first moment divided by the cell mass;
         stop when no centroid moves by more than ``tol``;
      3. make the result exactly antisymmetric, c_k = (c_k - c_{L-1-k}) / 2;
      4. per-coordinate MSE = E[y^2] - sum_k P_k c_k^2 with E[y^2] = 1/d,
         which holds because every centroid is its cell's mean.
    """
    if d < 3 or not (1 <= mse_bits <= 4):
        raise ValueError("need d >= 3 and 1 <= mse_bits <= 4")
    if tol is None:
        tol = 1e-13 / np.sqrt(d)   # ~5x above the float64 noise floor of one step
    L = 2 ** mse_bits
    c = coordinate_ppf((np.arange(L) + 0.5) / L, d) if init is None else np.array(init, np.float64)
    it = 0
    for it in range(1, max_iter + 1):
        t = np.concatenate(([-1.0], 0.5 * (c[:-1] + c[1:]), [1.0]))
        mass = coordinate_cdf(t[1:], d) - coordinate_cdf(t[:-1], d)
        new_c = cell_first_moment(t[:-1], t[1:], d) / mass
        moved = np.max(np.abs(new_c - c))
        c = new_c
        if moved < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    c = 0.5 * (c - c[::-1])
    t_inner = 0.5 * (c[:-1] + c[1:])
    t = np.concatenate(([-1.0], t_inner, [1.0]))
    mass = coordinate_cdf(t[1:], d) - coordinate_cdf(t[:-1], d)
    mse = 1.0 / d - float(np.sum(mass * c * c))
    return Codebook(d=d, mse_bits=mse_bits, centroids=c, boundaries=t_inner,
                    mse_per_coord=mse, iterations=it)

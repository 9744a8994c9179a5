"""Lloyd-Max codebooks on the rotated-coordinate marginal (oracle, fp64).

Sources (riverfrot "TurboQuant" post):
* section 4.1 — after x -> R x/|x| with a random orthogonal R, every
  coordinate follows the same Beta-type law that approaches a Gaussian as d
  grows;
* section 4.2 — Lloyd-Max (1-D k-means on a density) takes p(x) and 2^b
  levels and returns decision boundaries {t_i} and representatives {c_i};
  the codebook is computed once per (d, b) and only looked up at run time.

Reading taken where the pages are silent: the law is the exact marginal of
one coordinate of a uniform point on the unit sphere S^{d-1} (which is what
a Haar rotation of a fixed unit vector gives),

    f_d(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2),

i.e. (x+1)/2 ~ Beta((d-1)/2, (d-1)/2). Mean 0, variance 1/d. The Lloyd-Max
fixed point is unique for this log-concave density (d >= 3), so the start
point does not change the result.

Pinned by (tests/test_oracle_codebook.py): d = 3 uniform closed form;
1-bit closed form +-E|X|; dynamic-programming global optimum on a fine
grid for small d; symmetry; the pages' distortion bounds; Monte Carlo
variance and kurtosis of Haar-rotated unit vectors.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import betainc, gammaln


def _alpha(d: int) -> float:
    return (d - 1) / 2.0


def pdf(x, d: int):
    """f_d(x) on [-1, 1]."""
    x = np.asarray(x, dtype=np.float64)
    logc = gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)
    out = np.zeros_like(x)
    inside = np.abs(x) < 1.0
    out[inside] = np.exp(logc + (d - 3) / 2.0 * np.log1p(-x[inside] ** 2))
    if d == 3:
        out[np.abs(x) == 1.0] = 0.5
    return out


def cdf(x, d: int):
    """P(X <= x) via the regularised incomplete beta function."""
    x = np.clip(np.asarray(x, dtype=np.float64), -1.0, 1.0)
    a = _alpha(d)
    # Evaluate each half from its own tail so that no mass is lost to
    # cancellation against 1.
    lo = betainc(a, a, (x + 1.0) / 2.0)
    hi = 1.0 - betainc(a, a, (1.0 - x) / 2.0)
    return np.where(x <= 0.0, lo, hi)


def _cell_mass(a, b, d: int):
    """P(a <= X < b), evaluated from the tail each endpoint is nearer to."""
    al = _alpha(d)
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    # mirror so that both endpoints are <= 0 where that helps precision
    upper = a >= 0.0
    lo_mass = betainc(al, al, (b + 1.0) / 2.0) - betainc(al, al, (a + 1.0) / 2.0)
    up_mass = betainc(al, al, (1.0 - a) / 2.0) - betainc(al, al, (1.0 - b) / 2.0)
    return np.where(upper, up_mass, lo_mass)


def _first_moment(a, b, d: int):
    """Integral of x f_d(x) over [a, b] in closed form.

    d/dx (1-x^2)^((d-1)/2) = -(d-1) x (1-x^2)^((d-3)/2), so the integral is
    C [(1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)] / (d-1).
    """
    logc = gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)
    e = (d - 1) / 2.0

    def g(x):
        x = np.asarray(x, dtype=np.float64)
        return np.exp(e * np.log1p(-np.minimum(x * x, 1.0)))

    with np.errstate(divide="ignore"):
        return math.exp(logc) * (g(a) - g(b)) / (d - 1)


def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Lloyd-Max quantiser with 2^bits levels for f_d.

    Alternates the two optimality conditions until the centroids stop moving:
      thresholds: t_i = (c_{i-1} + c_i) / 2            (nearest-neighbour cells)
      centroids:  c_i = E[X | t_i <= X < t_{i+1}]       (conditional means)
    Returns (centroids [L], thresholds [L-1], D, iterations), ascending, where
    D = d * E[(X - Q(X))^2] is the total squared error of a unit vector.
    """
    if d < 3:
        raise ValueError("d must be >= 3")
    if not 1 <= bits <= 8:
        raise ValueError("bits out of range")
    L = 1 << bits
    # start from evenly spaced levels inside the support (the fixed point is
    # unique, so the start only affects the iteration count)
    span = min(2.0 / math.sqrt(d), 1.0 - 1.0 / L)
    c = np.linspace(-span, span, L)
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = _cell_mass(edges[:-1], edges[1:], d)
        m1 = _first_moment(edges[:-1], edges[1:], d)
        c_new = m1 / mass
        delta = np.max(np.abs(c_new - c))
        if not np.isfinite(delta):
            raise RuntimeError("Lloyd-Max iteration left the support")
        c = c_new
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    t = 0.5 * (c[:-1] + c[1:])
    D = distortion(c, t, d)
    return c, t, D, it


def _log_norm_const(d: int) -> float:
    return gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d - 1) / 2.0)


def _second_moment(a, b, d: int):
    """Integral of x^2 f_d(x) over [a, b], exactly.

    x^2 (1-x^2)^m = (1-x^2)^m - (1-x^2)^(m+1) with m = (d-3)/2, and
    (1-x^2)^(m+1) is the kernel of f_{d+2}; so the integral is
    P_d[a, b] - (C_d / C_{d+2}) P_{d+2}[a, b] with C the normalising constants.
    """
    ratio = math.exp(_log_norm_const(d) - _log_norm_const(d + 2))
    return _cell_mass(a, b, d) - ratio * _cell_mass(a, b, d + 2)


def distortion(centroids, thresholds, d: int) -> float:
    """d * E[(X - c[cell(X)])^2] = d * sum_i (M2_i - 2 c_i M1_i + c_i^2 P_i)."""
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], np.asarray(thresholds, dtype=np.float64), [1.0]))
    a, b = edges[:-1], edges[1:]
    P = _cell_mass(a, b, d)
    M1 = _first_moment(a, b, d)
    M2 = _second_moment(a, b, d)
    return float(d * np.sum(M2 - 2.0 * c * M1 + c * c * P))


def one_bit_centroid(d: int) -> float:
    """E|X| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)): the 1-bit Lloyd-Max level."""
    return math.exp(gammaln(d / 2.0) - 0.5 * math.log(math.pi) - gammaln((d + 1) / 2.0))


def brute_force_quantizer(d: int, levels: int, grid: int = 2000):
    """Globally optimal `levels`-cell quantiser of f_d on a discretised grid.

    Independent of the Lloyd iteration: exact dynamic programming over
    contiguous partitions of `grid` equal-width bins (each bin a point mass
    at its midpoint with its exact probability). Returns the centroids.
    """
    edges = np.linspace(-1.0, 1.0, grid + 1)
    p = np.diff(cdf(edges, d))
    x = 0.5 * (edges[:-1] + edges[1:])
    cp = np.concatenate(([0.0], np.cumsum(p)))
    cx = np.concatenate(([0.0], np.cumsum(p * x)))
    cxx = np.concatenate(([0.0], np.cumsum(p * x * x)))

    def cost(i, j):  # bins [i, j)
        w = cp[j] - cp[i]
        s = cx[j] - cx[i]
        return (cxx[j] - cxx[i]) - np.where(w > 0, s * s / np.where(w > 0, w, 1.0), 0.0)

    n = grid
    best = np.full((levels + 1, n + 1), np.inf)
    arg = np.zeros((levels + 1, n + 1), dtype=np.int64)
    best[0, 0] = 0.0
    idx = np.arange(n + 1)
    for k in range(1, levels + 1):
        for j in range(1, n + 1):
            i = idx[:j]
            v = best[k - 1, :j] + cost(i, j)
            a = int(np.argmin(v))
            best[k, j] = v[a]
            arg[k, j] = a
    cuts = [n]
    for k in range(levels, 0, -1):
        cuts.append(int(arg[k, cuts[-1]]))
    cuts = cuts[::-1]
    cents = []
    for k in range(levels):
        i, j = cuts[k], cuts[k + 1]
        cents.append((cx[j] - cx[i]) / (cp[j] - cp[i]))
    return np.array(cents)

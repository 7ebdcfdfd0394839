"""Lloyd-Max codebook for a rotated unit-vector coordinate (oracle, float64).

TurboQuant article §二, the coarse Lloyd-Max step (b−1 bits): after the key is
normalised and rotated, every coordinate follows the same (scaled Beta)
distribution; the quantiser is the continuous 1-D k-means (Lloyd-Max) solution
for that distribution, with 2**w levels, applied per coordinate by looking up
decision boundaries.

The distribution of one coordinate t of a uniform random point on the unit
sphere in R^d is the exact density

    f_d(t) = (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2),   t in [-1, 1],

equivalently (1 + t) / 2 ~ Beta((d-1)/2, (d-1)/2).  (The article calls it a
scaled Beta distribution that is close to N(0, 1/d) for large d; the exact
density is used here.)

Lloyd-Max alternates the two optimality conditions until they hold together:
  * boundaries are midpoints of neighbouring centroids;
  * each centroid is the conditional mean of its cell.
The cell probability is a regularised incomplete beta function and the cell's
first moment has the closed form
  int_u^v t f_d(t) dt = [(1-u^2)^(a+1) - (1-v^2)^(a+1)] / (2 (a+1) B(1/2,(d-1)/2)),
with a = (d-3)/2.
"""
from __future__ import annotations

import numpy as np
from scipy import special


def _log_norm(d: int) -> float:
    return special.betaln(0.5, (d - 1) / 2.0)


def cdf(t, d: int):
    """P(T <= t) for one coordinate of a uniform unit vector in R^d."""
    t = np.clip(np.asarray(t, dtype=np.float64), -1.0, 1.0)
    a = (d - 1) / 2.0
    return special.betainc(a, a, (1.0 + t) / 2.0)


def pdf(t, d: int):
    t = np.asarray(t, dtype=np.float64)
    a = (d - 3) / 2.0
    with np.errstate(invalid="ignore"):
        base = np.where(np.abs(t) < 1.0, 1.0 - t * t, 0.0)
        if a == 0.0:
            val = np.where(np.abs(t) <= 1.0, 1.0, 0.0)
        else:
            val = np.power(base, a)
    return val * np.exp(-_log_norm(d))


def _first_moment(u, v, d: int):
    """int_u^v t f_d(t) dt (closed form)."""
    a1 = (d - 3) / 2.0 + 1.0
    u = np.clip(u, -1.0, 1.0)
    v = np.clip(v, -1.0, 1.0)
    fu = np.power(1.0 - u * u, a1)
    fv = np.power(1.0 - v * v, a1)
    return (fu - fv) / (2.0 * a1) * np.exp(-_log_norm(d))


def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000,
              init=None, symmetric: bool = True):
    """Lloyd-Max quantiser of f_d with 2**bits levels.

    Returns (centroids[2**bits], boundaries[2**bits - 1], iterations) in float64,
    both ascending.  The default start point is the distribution's
    mid-quantiles; f_d is log-concave for d >= 3, so the fixed point does not
    depend on it.  f_d is even, so the fixed point is odd-symmetric; with
    ``symmetric`` each iterate is symmetrised (c <- (c - reversed(c)) / 2),
    which keeps the middle boundary exactly 0 instead of a rounding residue.
    """
    if bits < 1:
        raise ValueError("bits must be >= 1")
    if d < 3:
        raise ValueError("d must be >= 3")
    L = 1 << bits
    if init is None:
        p = (np.arange(L) + 0.5) / L
        a = (d - 1) / 2.0
        c = 2.0 * special.betaincinv(a, a, p) - 1.0
    else:
        c = np.sort(np.asarray(init, dtype=np.float64))
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = np.diff(cdf(edges, d))
        mom = _first_moment(edges[:-1], edges[1:], d)
        c_new = mom / mass
        if symmetric:
            c_new = 0.5 * (c_new - c_new[::-1])
        delta = np.max(np.abs(c_new - c))
        c = c_new
        if delta < tol:
            break
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def distortion(d: int, centroids, boundaries) -> float:
    """E[(T - Q(T))^2] for the quantiser (centroids, boundaries) under f_d,
    by adaptive quadrature of (t - c_k)^2 f_d(t) over each cell."""
    from scipy import integrate

    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate(([-1.0], np.asarray(boundaries, dtype=np.float64), [1.0]))
    total = 0.0
    for k in range(len(c)):
        lo, hi = edges[k], edges[k + 1]
        val, _ = integrate.quad(lambda x: (x - c[k]) ** 2 * pdf(x, d), lo, hi,
                                epsabs=1e-15, epsrel=1e-12, limit=200,
                                points=[0.0] if lo < 0.0 < hi else None)
        total += val
    return total


def codebook_fp32(d: int, bits: int):
    """The codebook as stored and handed to both sides: fp32 centroids and
    boundaries (boundaries are the fp32 rounding of the float64 midpoints)."""
    c, t, _ = lloyd_max(d, bits)
    return c.astype(np.float32), t.astype(np.float32)

"""Lloyd-Max codebook for one coordinate of a uniformly rotated unit vector (oracle, fp64).

Source: "TurboQuant: ... MNN on phones", section 2.2 (after a uniform random rotation a
coordinate of a point on the unit sphere in R^dim has density proportional to
(1 - t^2)^((dim-3)/2) on [-1, 1]) and section 2.3 (Lloyd-Max = one-dimensional
continuous k-means on that law: 2^b cells, centroid = probability-weighted mean of the
cell, boundary = midpoint of neighbouring centroids, iterate to convergence, integrals
done numerically).

Reading taken where the page is loose: the page's geometric aside in 2.2 gives the
exponent (dim-2)/2, while its displayed formula gives (dim-3)/2.  The displayed formula
is used; its variance is exactly 1/dim, which is what 2.2 (and "RotaryQuant", key
design 2) state.  ``dim`` is the size of the normalised group (32 for the block-32
transform, 128 for a whole-head rotation), because it is the group that lies on a
sphere.
"""

from functools import lru_cache

import numpy as np
from scipy import integrate, special


def density(t, dim):
    """f(t) = (1 - t^2)^((dim-3)/2) / B(1/2, (dim-1)/2) for t in [-1, 1] (2.2)."""
    t = np.asarray(t, dtype=np.float64)
    out = np.zeros_like(t)
    inside = np.abs(t) < 1.0
    out[inside] = (1.0 - t[inside] ** 2) ** ((dim - 3) / 2.0) / special.beta(0.5, (dim - 1) / 2.0)
    return out


def _f(t, dim):
    return (1.0 - t * t) ** ((dim - 3) / 2.0) / special.beta(0.5, (dim - 1) / 2.0)


def _cell_moments(lo, hi, dim):
    """(mass, first moment) of the law on [lo, hi] by adaptive quadrature; in 2 dimensions
    (the arcsine law 1 / (pi sqrt(1 - t^2)), singular at the ends) by its closed forms."""
    if dim == 2:
        return ((np.arcsin(hi) - np.arcsin(lo)) / np.pi,
                (np.sqrt(max(0.0, 1.0 - lo * lo)) - np.sqrt(max(0.0, 1.0 - hi * hi))) / np.pi)
    m0 = integrate.quad(_f, lo, hi, args=(dim,), epsabs=1e-16, epsrel=1e-13, limit=200)[0]
    m1 = integrate.quad(lambda t: t * _f(t, dim), lo, hi, epsabs=1e-16, epsrel=1e-13, limit=200)[0]
    return m0, m1


@lru_cache(maxsize=None)
def _lloyd_max_cached(bits, dim):
    if bits < 1 or dim < 2:
        raise ValueError("bits >= 1 and dim >= 2 are required")
    n = 2 ** bits
    # start from evenly spaced levels over +-2 standard deviations (std = 1/sqrt(dim)),
    # kept inside (-1, 1) for the smallest dimensions
    c = np.linspace(-2.0, 2.0, n) / np.sqrt(dim)
    if dim < 4:
        c = np.linspace(-0.9, 0.9, n)
    for _ in range(100000):
        m = 0.5 * (c[:-1] + c[1:])                     # boundary = midpoint (2.3)
        edges = np.concatenate([[-1.0], m, [1.0]])
        new = np.empty(n)
        for k in range(n):                             # centroid = conditional mean (2.3)
            m0, m1 = _cell_moments(edges[k], edges[k + 1], dim)
            new[k] = m1 / m0
        delta = np.max(np.abs(new - c))
        c = new
        if delta < 1e-14:
            break
    else:  # pragma: no cover - convergence is fast for every supported (bits, dim)
        raise RuntimeError("Lloyd-Max iteration did not converge")
    # The law is even in t (2.2), so the fixed point is odd-symmetric; fold away the
    # last-bit asymmetry of the quadrature so that the middle boundary is exactly 0 (it
    # decides the code of an exact zero coordinate).
    c = 0.5 * (c - c[::-1])
    m = 0.5 * (c[:-1] + c[1:])
    return c, m


def lloyd_max(bits, dim):
    """Return (centroids[2^bits], boundaries[2^bits - 1]) in float64, ascending.

    Converged Lloyd-Max quantiser for ``density(., dim)``; boundaries are the midpoints
    of neighbouring centroids (2.3).
    """
    c, m = _lloyd_max_cached(int(bits), int(dim))
    return c.copy(), m.copy()


def distortion(bits, dim):
    """D1 = E[(t - Q(t))^2] under the coordinate law, by quadrature per cell.

    For a unit vector rotated uniformly, the expected squared error of the whole
    reconstructed group is dim * D1 (sum over dim identically distributed coordinates),
    the quantity bounded by 2.7 / 4^b in 2.3.
    """
    c, m = lloyd_max(bits, dim)
    edges = np.concatenate([[-1.0], m, [1.0]])
    total = 0.0
    for k in range(len(c)):
        total += integrate.quad(lambda t: (t - c[k]) ** 2 * _f(t, dim), edges[k], edges[k + 1],
                                epsabs=1e-16, epsrel=1e-12, limit=200)[0]
    return total

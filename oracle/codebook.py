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
from scipy import integrate, linalg, special


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


def _cell_moments_closed(lo, hi, dim):
    """(mass, first moment) of the law on every cell [lo[k], hi[k]] in closed form: the mass
    from the CDF F(t) = I_{(1+t)/2}(a, a), a = (dim-1)/2 (t^2 of a sphere coordinate is
    Beta(1/2, a)), taken from the nearer end so that tail cells keep their digits; the first
    moment from the primitive -(1-t^2)^a / (2a B(1/2, a)), differenced through expm1."""
    a = (dim - 1) / 2.0
    lo, hi = np.asarray(lo, dtype=np.float64), np.asarray(hi, dtype=np.float64)
    up = lo >= 0.0
    m0 = np.where(up, special.betainc(a, a, (1.0 - lo) / 2.0) - special.betainc(a, a, (1.0 - hi) / 2.0),
                  special.betainc(a, a, (1.0 + hi) / 2.0) - special.betainc(a, a, (1.0 + lo) / 2.0))
    with np.errstate(divide="ignore", invalid="ignore"):
        L, H = a * np.log1p(-lo * lo), a * np.log1p(-hi * hi)  # log (1 - t^2)^a at the ends
        diff = np.where(L >= H, -np.exp(L) * np.expm1(H - L), np.exp(H) * np.expm1(L - H))
    diff = np.where(np.isneginf(L) & np.isneginf(H), 0.0, diff)
    return m0, diff / (2.0 * a * special.beta(0.5, a))


@lru_cache(maxsize=None)
def _lloyd_max_newton(bits, dim):
    """The same fixed point for 32 to 256 levels, where the plain iteration above converges
    too slowly: Newton's method on c_k - E[t | cell k] = 0 (the conditions of 2.3), whose
    Jacobian is tridiagonal because cell k's mean depends on c_{k-1}, c_k, c_{k+1} through
    its two boundaries (d/db of the cell integrals: the density at b, and b times it).  The
    start puts levels at the quantiles of the density^(1/3) law, the asymptotic point
    density of optimal quantisers (Panter and Dite); steps are halved until the levels stay
    ordered inside (-1, 1)."""
    n = 2 ** bits
    grid = np.linspace(-1.0, 1.0, 400001)[1:-1]
    g = density(grid, dim) ** (1.0 / 3.0)
    cum = np.concatenate([[0.0], np.cumsum(0.5 * (g[1:] + g[:-1]) * np.diff(grid))])
    c = np.interp((np.arange(n) + 0.5) / n, cum / cum[-1], grid)
    for _ in range(200):
        b = 0.5 * (c[:-1] + c[1:])
        m0, m1 = _cell_moments_closed(np.concatenate([[-1.0], b]), np.concatenate([b, [1.0]]), dim)
        mean = m1 / m0
        resid = c - mean
        if np.max(np.abs(resid)) < 1e-13:  # the moments' own rounding is about 1e-14
            break
        fb = density(b, dim)
        # d mean_k / d b = (b - mean_k) f(b) / m0_k at its upper boundary, minus that at its
        # lower one; each boundary moves by half of either neighbouring level
        up_term = (b - mean[:-1]) * fb / (2.0 * m0[:-1])   # cell k, its upper boundary b_k
        lo_term = (b - mean[1:]) * fb / (2.0 * m0[1:])     # cell k + 1, its lower boundary b_k
        band = np.zeros((3, n))
        band[1] = 1.0
        band[1, :-1] -= up_term
        band[1, 1:] += lo_term
        band[0, 1:] = -up_term
        band[2, :-1] = lo_term
        step = linalg.solve_banded((1, 1), band, resid)
        lam = 1.0
        while True:
            new = c - lam * step
            if np.all(np.diff(new) > 0) and new[0] > -1.0 and new[-1] < 1.0:
                break
            lam *= 0.5
        c = new
    else:  # pragma: no cover
        raise RuntimeError("Lloyd-Max Newton iteration did not converge")
    c = 0.5 * (c - c[::-1])  # odd symmetry, as above
    return c, 0.5 * (c[:-1] + c[1:])


def lloyd_max(bits, dim):
    """Return (centroids[2^bits], boundaries[2^bits - 1]) in float64, ascending.

    Converged Lloyd-Max quantiser for ``density(., dim)``; boundaries are the midpoints
    of neighbouring centroids (2.3).  1 to 4 bits by the plain iteration, 5 to 8 bits (the
    byte containers of "RoPE-Aware Bit Allocation ...") by Newton's method on the same
    conditions.
    """
    bits, dim = int(bits), int(dim)
    if bits > 8:
        raise ValueError("at most 8 bits")
    c, m = _lloyd_max_cached(bits, dim) if bits <= 4 else _lloyd_max_newton(bits, dim)
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

"""Pins for the oracle's coordinate law and Lloyd-Max codebook.

Each check ties the oracle to something other than itself: closed forms (moments of the
law, incomplete-beta cell masses), the definition of the law (coordinates of uniform
points on the sphere), a textbook table (Gaussian Lloyd-Max levels, the large-dim limit)
and the bounds the pages print ("TurboQuant ... MNN on phones", 2.2-2.4).
"""

import json
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

from oracle import codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLDEN, "page_facts.json")))
CASES = [(3, 32), (4, 32), (3, 128), (4, 128)]


def beta_cdf(t, dim):
    """Closed-form CDF of the coordinate law: F(t) = I_{(1+t)/2}((dim-1)/2, (dim-1)/2)."""
    a = (dim - 1) / 2.0
    return special.betainc(a, a, (1.0 + np.asarray(t)) / 2.0)


def first_moment(lo, hi, dim):
    """Closed form of int_lo^hi t f(t) dt = [-(1-t^2)^(mu+1) / (2(mu+1))] / B(1/2, (dim-1)/2)."""
    mu = (dim - 3) / 2.0
    prim = lambda t: -(1.0 - t * t) ** (mu + 1) / (2.0 * (mu + 1))
    return (prim(hi) - prim(lo)) / special.beta(0.5, (dim - 1) / 2.0)


@pytest.mark.parametrize("dim", [3, 8, 32, 128, 1024])
def test_density_normalised_and_variance_is_one_over_dim(dim):
    # 2.2: the law's variance tends to 1/dim; with the displayed exponent (dim-3)/2 it is
    # exactly 1/dim, which rules out the aside's (dim-2)/2 (variance 1/(dim+1)).
    mass = integrate.quad(lambda t: codebook.density(np.array([t]), dim)[0], -1, 1, epsabs=1e-14)[0]
    var = integrate.quad(lambda t: t * t * codebook.density(np.array([t]), dim)[0], -1, 1, epsabs=1e-15)[0]
    assert abs(mass - 1.0) < 1e-10
    assert abs(var * dim - 1.0) < 1e-9


def test_density_std_at_head_dim_matches_page():
    std = np.sqrt(integrate.quad(lambda t: t * t * codebook.density(np.array([t]), 128)[0], -1, 1)[0])
    assert abs(std - FACTS["coordinate_std_d128"]["value"]) < 5e-4


@pytest.mark.parametrize("dim", [32, 128])
def test_density_is_law_of_sphere_coordinate(dim):
    # Definition (2.2): a coordinate of a uniform point on S^{dim-1}.  Sample by
    # normalising Gaussian vectors and compare with the oracle density's CDF (quadrature).
    rng = np.random.default_rng(1234)
    x = rng.standard_normal((200000, dim))
    t = x[:, 0] / np.linalg.norm(x, axis=1)
    grid = np.linspace(-0.6, 0.6, 13) * (1 if dim == 32 else 0.5)
    for g in grid:
        cdf_quad = integrate.quad(lambda s: codebook.density(np.array([s]), dim)[0], -1, g, epsabs=1e-14)[0]
        assert abs(cdf_quad - beta_cdf(g, dim)) < 1e-10          # closed form
        assert abs(np.mean(t <= g) - cdf_quad) < 4e-3            # sampling error ~1e-3
    assert stats.kstest(t, lambda s: beta_cdf(s, dim)).pvalue > 1e-3


@pytest.mark.parametrize("bits,dim", CASES)
def test_lloyd_max_fixed_point_closed_form(bits, dim):
    # 2.3: every centroid is the conditional mean of its cell, every boundary the
    # midpoint.  Cell mass from the incomplete beta function, numerator in closed form.
    c, m = codebook.lloyd_max(bits, dim)
    assert c.shape == (2 ** bits,) and m.shape == (2 ** bits - 1,)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_allclose(m, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    edges = np.concatenate([[-1.0], m, [1.0]])
    for k in range(2 ** bits):
        mass = beta_cdf(edges[k + 1], dim) - beta_cdf(edges[k], dim)
        cond_mean = first_moment(edges[k], edges[k + 1], dim) / mass
        assert abs(cond_mean - c[k]) < 1e-12 * max(1.0, abs(c[k]) * np.sqrt(dim))


@pytest.mark.parametrize("bits,dim", CASES)
def test_lloyd_max_symmetric(bits, dim):
    c, m = codebook.lloyd_max(bits, dim)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-14)
    assert abs(m[len(m) // 2]) < 1e-14


@pytest.mark.parametrize("levels", [8, 16])
def test_large_dim_limit_is_gaussian_lloyd_max(levels):
    # 2.2: at high dimension the law is N(0, 1/dim), so sqrt(dim)*c tends to the Gaussian
    # Lloyd-Max levels (Max 1960, tests/golden/gaussian_lloyd_max.txt).
    rows = {}
    for line in open(os.path.join(GOLDEN, "gaussian_lloyd_max.txt")):
        if line.strip() and not line.startswith("#"):
            parts = line.split()
            rows[int(parts[0])] = np.array([float(v) for v in parts[1:]])
    bits = int(np.log2(levels))
    dim = 20000
    c, _ = codebook.lloyd_max(bits, dim)
    half = np.sqrt(dim) * c[levels // 2:]
    np.testing.assert_allclose(half, rows[levels], atol=2e-3)
    # and the approach is monotone in dim: 128 is closer than 32
    err = [np.max(np.abs(np.sqrt(d) * codebook.lloyd_max(bits, d)[0][levels // 2:] - rows[levels]))
           for d in (32, 128)]
    assert err[1] < err[0]


@pytest.mark.parametrize("bits,dim", [(3, 32), (3, 128), (4, 32), (4, 128)])
def test_centroids_are_cell_means_of_sphere_coordinates(bits, dim):
    # 2.3: each centroid is the probability-weighted mean of its cell.  Check it on
    # coordinates of uniform points on the sphere (the law's definition, 2.2), sampled
    # independently of the density formula: per cell, the sample mean must match the
    # oracle centroid within its standard error, and the cell's sample mass must match
    # the incomplete-beta mass.
    rng = np.random.default_rng(99)
    x = rng.standard_normal((40000, dim))
    t = (x / np.linalg.norm(x, axis=1, keepdims=True)).ravel()
    c, m = codebook.lloyd_max(bits, dim)
    cell = np.searchsorted(m, t)
    edges = np.concatenate([[-1.0], m, [1.0]])
    for k in range(2 ** bits):
        s = t[cell == k]
        se = s.std() / np.sqrt(len(s))
        assert abs(s.mean() - c[k]) < 5 * se
        mass = beta_cdf(edges[k + 1], dim) - beta_cdf(edges[k], dim)
        assert abs(len(s) / len(t) - mass) < 5 * np.sqrt(mass * (1 - mass) / len(t)) * 2


@pytest.mark.parametrize("bits,dim", CASES)
def test_mse_within_page_bounds(bits, dim):
    # 2.3: unit-vector MSE <= 2.7 / 4^b and above the 1 / 4^b lower bound.
    mse = dim * codebook.distortion(bits, dim)
    assert FACTS["mse_lower_constant"]["value"] / 4 ** bits < mse < FACTS["mse_upper_constant"]["value"] / 4 ** bits


@pytest.mark.parametrize("bits,dim", CASES)
def test_inner_product_shrink_matches_page(bits, dim):
    # 2.4: an MSE quantiser shrinks inner products, about 4% at 3 bits and 1% at 4 bits.
    # With centroid cells E[t Q(t)] = E[Q(t)^2] = E[t^2] - D1, so the shrink of <x, x_hat>
    # for a unit x is dim * D1.  Compare with the printed rounded figures.
    shrink = dim * codebook.distortion(bits, dim)
    target = FACTS["inner_product_shrink_3bit" if bits == 3 else "inner_product_shrink_4bit"]["value"]
    assert abs(shrink - target) < 0.5 * target


# ---- 5 to 8 bits (byte containers of "RoPE-Aware Bit Allocation ..."): Newton's method on
# the same fixed-point conditions

WIDE = [(5, 2), (5, 8), (6, 32), (7, 4), (8, 2), (8, 16), (8, 128)]


def cell_mass(lo, hi, dim):
    """Incomplete-beta mass of [lo, hi], from the nearer tail (F(-t) = 1 - F(t))."""
    return beta_cdf(-lo, dim) - beta_cdf(-hi, dim) if lo >= 0 else beta_cdf(hi, dim) - beta_cdf(lo, dim)


@pytest.mark.parametrize("bits,dim", WIDE)
def test_wide_lloyd_max_fixed_point_closed_form(bits, dim):
    c, m = codebook.lloyd_max(bits, dim)
    assert c.shape == (2 ** bits,) and np.all(np.diff(c) > 0) and -1 < c[0] and c[-1] < 1
    np.testing.assert_allclose(m, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-16)
    np.testing.assert_allclose(c, -c[::-1], atol=1e-15)
    edges = np.concatenate([[-1.0], m, [1.0]])
    for k in range(2 ** bits):
        cond_mean = first_moment(edges[k], edges[k + 1], dim) / cell_mass(edges[k], edges[k + 1], dim)
        assert abs(cond_mean - c[k]) < 1e-11 * max(1.0, abs(c[k]) * np.sqrt(dim)), k


@pytest.mark.parametrize("bits,dim", [(3, 32), (4, 128), (3, 2), (4, 8)])
def test_newton_equals_the_plain_iteration(bits, dim):
    # two methods, one fixed point: the 5-8-bit solver run at 3-4 bits
    c_newton, _ = codebook._lloyd_max_newton(bits, dim)
    c_plain, _ = codebook.lloyd_max(bits, dim)
    np.testing.assert_allclose(c_newton, c_plain, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dim", [8, 32, 128])
def test_wide_mse_bounds_and_high_rate_limit(dim):
    # 2.3: dim * D1 <= 2.7 / 4^b at every width, and at high rate dim * D1 * 4^b rises
    # towards the Panter-Dite constant dim / 12 * (int f^(1/3))^3 (written out by quadrature)
    pd = dim / 12.0 * integrate.quad(lambda t: codebook.density(np.array([t]), dim)[0] ** (1 / 3), -1, 1,
                                     epsabs=1e-13, limit=400)[0] ** 3
    scaled = [dim * codebook.distortion(b, dim) * 4 ** b for b in (5, 6, 7, 8)]
    assert all(s < FACTS["mse_upper_constant"]["value"] for s in scaled)
    assert all(x < y for x, y in zip(scaled, scaled[1:])) and scaled[-1] < pd
    assert pd - scaled[-1] < 0.015 * pd


def test_wide_centroids_are_cell_means_of_sphere_coordinates():
    rng = np.random.default_rng(98)
    dim, bits = 8, 5
    x = rng.standard_normal((200000, dim))
    t = (x / np.linalg.norm(x, axis=1, keepdims=True)).ravel()
    c, m = codebook.lloyd_max(bits, dim)
    cell = np.searchsorted(m, t)
    for k in range(2 ** bits):
        s = t[cell == k]
        assert abs(s.mean() - c[k]) < 5 * s.std() / np.sqrt(len(s)), k

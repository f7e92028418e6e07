"""Pins for the oracle quantiser/dequantiser ("TurboQuant ... MNN on phones", 2.1-2.4, 3.4).

* search: the compare-count rule equals a library binary search and, by the midpoint
  boundaries, the brute-force nearest centroid; exact ties take the lower code;
* quantise -> dequantise of isotropic vectors reproduces the exact expected error
  dim * D1 per group (any dropped term, wrong sign or non-orthogonal step breaks it);
* norms are the group L2 norms, zero groups map to the code of 0 and dequantise to 0;
  scaling by a power of two scales only the norms.
"""

import numpy as np
import pytest

from oracle import codebook, quant, rotation


def unit_quats(rng, shape):
    q = rng.standard_normal(shape + (4,))
    return q / np.linalg.norm(q, axis=-1, keepdims=True)


@pytest.mark.parametrize("bits,dim", [(3, 32), (4, 128)])
def test_search_rule(bits, dim):
    c, m = codebook.lloyd_max(bits, dim)
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.standard_normal(20000) / np.sqrt(dim), m, [-1.0, 1.0, 0.0, -np.inf, np.inf]])
    idx = quant.search(y, m)
    np.testing.assert_array_equal(idx, np.searchsorted(m, y, side="left"))
    # exact boundary values take the lower code (count of boundaries strictly below)
    np.testing.assert_array_equal(quant.search(m, m), np.arange(len(m)))
    # away from ties the rule is the nearest centroid (brute force over all centroids)
    away = y[np.isfinite(y) & (quant.boundary_distance(y, m) > 1e-12)]
    np.testing.assert_array_equal(quant.search(away, m), np.argmin(np.abs(away[:, None] - c), axis=1))


@pytest.mark.parametrize("bits,group,use_so4", [(3, 32, False), (4, 32, False), (3, 128, True), (4, 128, False)])
def test_reconstruction_error_equals_exact_distortion(bits, group, use_so4):
    # For isotropic x the rotated normalised group is uniform on the sphere, so
    # E||x_hat - dequant||^2 / ||x||^2 = group * D1 exactly (2.3); Monte Carlo within 4 SE.
    rng = np.random.default_rng(6)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    so4 = unit_quats(rng, (32, 2)) if use_so4 else None
    c, m = codebook.lloyd_max(bits, group)
    x = rng.standard_normal((4000, 128))
    idx, norms, y = quant.quantize(x, signs, group, c, m, so4)
    xt = quant.dequantize(idx, norms, signs, group, c, so4)
    ng = 128 // group
    err = np.sum(((x - xt).reshape(-1, ng, group)) ** 2, axis=-1) / np.sum(x.reshape(-1, ng, group) ** 2, axis=-1)
    expect = group * codebook.distortion(bits, group)
    assert abs(err.mean() - expect) < 4 * err.std() / np.sqrt(err.size)
    # y really is R(x / ||x_grp||): rows have unit group norm and undo to x
    np.testing.assert_allclose(np.sum(y.reshape(-1, ng, group) ** 2, axis=-1), 1.0, atol=1e-12)
    xr = rotation.unrotate(y, signs, group, so4).reshape(-1, ng, group) * norms[..., None].astype(np.float64)
    np.testing.assert_allclose(xr.reshape(x.shape), x, rtol=2e-7, atol=2e-6)
    # the inner-product shrink of 2.4 on the same samples
    unit = x.reshape(-1, ng, group) / np.linalg.norm(x.reshape(-1, ng, group), axis=-1, keepdims=True)
    recon = quant.dequantize(idx, np.ones_like(norms), signs, group, c, so4).reshape(-1, ng, group)
    shrink = 1.0 - np.sum(unit * recon, axis=-1)
    assert abs(shrink.mean() - expect) < 4 * shrink.std() / np.sqrt(shrink.size)


def test_norms_zero_groups_and_scaling():
    rng = np.random.default_rng(7)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    c, m = codebook.lloyd_max(3, 32)
    x = rng.standard_normal((3, 128)).astype(np.float32)
    x[1, 32:64] = 0.0
    x[2] = 0.0
    idx, norms, _ = quant.quantize(x, signs, 32, c, m)
    np.testing.assert_array_equal(norms, np.linalg.norm(x.astype(np.float64).reshape(3, 4, 32), axis=-1).astype(np.float32))
    assert norms.dtype == np.float32
    zero_code = int(np.sum(m < 0))
    assert zero_code == 3
    assert np.all(idx[1, 32:64] == zero_code) and np.all(idx[2] == zero_code)
    xt = quant.dequantize(idx, norms, signs, 32, c)
    assert np.all(xt[1, 32:64] == 0.0) and np.all(xt[2] == 0.0)
    idx4, norms4, _ = quant.quantize(4.0 * x, signs, 32, c, m)
    np.testing.assert_array_equal(idx4, idx)
    np.testing.assert_array_equal(norms4, 4.0 * norms)


def test_per_group_independence():
    # each 32-block is normalised and rotated on its own (3.1): changing one block leaves
    # the other blocks' codes and norms untouched
    rng = np.random.default_rng(8)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    c, m = codebook.lloyd_max(3, 32)
    x = rng.standard_normal(128)
    x2 = x.copy()
    x2[64:96] = rng.standard_normal(32) * 5
    i1, n1, _ = quant.quantize(x, signs, 32, c, m)
    i2, n2, _ = quant.quantize(x2, signs, 32, c, m)
    keep = np.r_[0:64, 96:128]
    np.testing.assert_array_equal(i1[keep], i2[keep])
    np.testing.assert_array_equal(n1[[0, 1, 3]], n2[[0, 1, 3]])

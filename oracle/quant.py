"""Quantise / dequantise one head vector per (token, KV head) (oracle, fp64).

Source: "TurboQuant: ... MNN on phones", 2.1 (three steps: norm = ||x||_2 and x_hat =
x / norm; y = Pi x_hat; indices[i] = codebook_search(y[i]); dequantisation is lookup ->
inverse rotation -> times norm), 3.1 (one L2 norm per 32-dimensional block) and 3.4
(the search is a count of "greater than" comparisons against the boundaries).

Readings:
* the norm group equals the rotation block g (32, or the whole head of 128 for the
  IsoQuant rotation), and the codebook is derived for dimension g;
* a zero group stores norm 0; its normalised vector is taken as 0, which maps to code
  #{boundaries < 0} and dequantises to 0;
* idx = #{k : y > m_k}, so a value exactly on a boundary takes the lower code;
* the stored norm is fp32, rounded to nearest from the fp64 norm; dequantisation uses
  that stored value and the fp64 codebook, with no renormalisation.
"""

import numpy as np

from . import rotation


def search(y, boundaries):
    """Code index = number of boundaries strictly below y (compare-count rule, 3.4)."""
    y = np.asarray(y, dtype=np.float64)
    idx = np.zeros(y.shape, dtype=np.int64)
    for m in np.asarray(boundaries, dtype=np.float64):
        idx += (y > m)
    return idx.astype(np.uint8)


def quantize(x, signs, group, centroids, boundaries, so4=None):
    """Quantise x[..., d] (one KV head's rotation) into codes and fp32 group norms.

    Returns (idx uint8[..., d], norms float32[..., d/group], y float64[..., d]) where y is
    the rotated normalised vector whose coordinates were searched (kept so that tests can
    measure each coordinate's distance to the nearest boundary).
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ng = d // group
    xg = x.reshape(x.shape[:-1] + (ng, group))
    n = np.sqrt(np.sum(xg * xg, axis=-1))                      # step 1: group L2 norm
    safe = np.where(n > 0, n, 1.0)
    xhat = np.where(n[..., None] > 0, xg / safe[..., None], 0.0).reshape(x.shape)
    y = rotation.rotate(xhat, signs, group, so4)                # step 2: rotate
    idx = search(y, boundaries)                                  # step 3: scalar search
    return idx, n.astype(np.float32), y


def dequantize(idx, norms, signs, group, centroids, so4=None):
    """x_tilde = norm * R^T c[idx], per group (2.1: lookup -> inverse rotation -> times norm)."""
    c = np.asarray(centroids, dtype=np.float64)[np.asarray(idx, dtype=np.int64)]
    x = rotation.unrotate(c, signs, group, so4)
    d = x.shape[-1]
    ng = d // group
    xg = x.reshape(x.shape[:-1] + (ng, group)) * np.asarray(norms, dtype=np.float64)[..., None]
    return xg.reshape(x.shape)


def boundary_distance(y, boundaries):
    """min_k |y - m_k| for every coordinate (fp64), for the near-boundary parity rule."""
    y = np.asarray(y, dtype=np.float64)
    m = np.asarray(boundaries, dtype=np.float64)
    return np.min(np.abs(y[..., None] - m), axis=-1)

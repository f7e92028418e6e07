"""Orthogonal rotation R applied to keys, values and queries (oracle, fp64).

R = S_SO4 . H . D_s, applied in that order to a head vector x (length head_dim):

1. D_s: multiply coordinate i by the per-KV-head sign s_i in {+1, -1} ("TurboQuant ...
   MNN on phones", 3.1: deterministic +-1 sign flips give the Hadamard transform the
   randomness the method needs).  The page generates the signs with a hash it does not
   give; here they are an explicit seeded input array.
2. H: the normalised Walsh-Hadamard matrix H_g / sqrt(g) in Sylvester (natural) order on
   each contiguous block of g coordinates (3.1: blocks of 32 with 5 butterfly stages;
   "RotaryQuant ...", key design 2: the whole head, H_d).
3. S_SO4 (optional, IsoQuant): each contiguous 4-block v (read as the quaternion
   v0 + v1 i + v2 j + v3 k) becomes q_L v conj(q_R) with unit quaternions q_L, q_R
   ("RotaryQuant ...", key design 2; R = R_SO(4) o H_d, i.e. the Hadamard first).

R^T applies the inverses in reverse order: v = conj(q_L) w q_R, then H (symmetric and
its own inverse once normalised), then the signs.  The oracle forms H explicitly and
multiplies; no butterfly, blocking or fusion.
"""

import numpy as np


def hadamard(g):
    """Normalised Sylvester Hadamard matrix H_g / sqrt(g), built by H_2n = [[H, H], [H, -H]]."""
    if g < 1 or (g & (g - 1)) != 0:
        raise ValueError("g must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(g)


def qmul(p, q):
    """Hamilton product of quaternions stored as [..., 4] = (real, i, j, k)."""
    a1, b1, c1, d1 = np.moveaxis(np.asarray(p, dtype=np.float64), -1, 0)
    a2, b2, c2, d2 = np.moveaxis(np.asarray(q, dtype=np.float64), -1, 0)
    return np.stack([
        a1 * a2 - b1 * b2 - c1 * c2 - d1 * d2,
        a1 * b2 + b1 * a2 + c1 * d2 - d1 * c2,
        a1 * c2 - b1 * d2 + c1 * a2 + d1 * b2,
        a1 * d2 + b1 * c2 - c1 * b2 + d1 * a2,
    ], axis=-1)


def qconj(q):
    q = np.asarray(q, dtype=np.float64)
    return q * np.array([1.0, -1.0, -1.0, -1.0])


def so4_forward(x, so4):
    """Apply v -> q_L v conj(q_R) to every 4-block of x[..., d]; so4 is [d/4, 2, 4] (q_L, q_R)."""
    d = x.shape[-1]
    v = x.reshape(x.shape[:-1] + (d // 4, 4))
    ql = so4[:, 0, :]
    qr = so4[:, 1, :]
    w = qmul(qmul(ql, v), qconj(qr))
    return w.reshape(x.shape)


def so4_inverse(x, so4):
    """Inverse of ``so4_forward``: w -> conj(q_L) w q_R (unit quaternions)."""
    d = x.shape[-1]
    w = x.reshape(x.shape[:-1] + (d // 4, 4))
    ql = so4[:, 0, :]
    qr = so4[:, 1, :]
    v = qmul(qmul(qconj(ql), w), qr)
    return v.reshape(x.shape)


def _block_hadamard(x, g):
    d = x.shape[-1]
    h = hadamard(g)
    xb = x.reshape(x.shape[:-1] + (d // g, g))
    return (xb @ h.T).reshape(x.shape)


def rotate(x, signs, group, so4=None):
    """y = R x for x[..., d] with one KV head's signs[d] (and so4[d/4, 2, 4] or None)."""
    x = np.asarray(x, dtype=np.float64)
    y = x * np.asarray(signs, dtype=np.float64)
    y = _block_hadamard(y, group)
    if so4 is not None:
        y = so4_forward(y, np.asarray(so4, dtype=np.float64))
    return y


def unrotate(y, signs, group, so4=None):
    """x = R^T y, the exact inverse of ``rotate``."""
    y = np.asarray(y, dtype=np.float64)
    if so4 is not None:
        y = so4_inverse(y, np.asarray(so4, dtype=np.float64))
    x = _block_hadamard(y, group)          # H / sqrt(g) is symmetric and orthogonal
    return x * np.asarray(signs, dtype=np.float64)


def rotation_matrix(signs, group, so4=None):
    """Dense R (d x d) for one head, column j = R e_j (used by pins and the rotated-domain check)."""
    d = len(signs)
    return rotate(np.eye(d), signs, group, so4).T

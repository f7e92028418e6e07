"""Pins for the oracle's rotation R = S_SO4 . H . D_s and its inverse.

Checked against a library Hadamard (scipy.linalg.hadamard), the quaternion multiplication
table (i j = k, ...), an independent 4x4-matrix form of v -> q_L v conj(q_R), and the
facts "RotaryQuant ..." states in key design 2 (orthogonality, 6 degrees of freedom, the
25% fixed subspace of a single-quaternion rotation, operation and parameter counts).
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import rotation

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def unit_quats(rng, shape):
    q = rng.standard_normal(shape + (4,))
    return q / np.linalg.norm(q, axis=-1, keepdims=True)


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_matches_library(g):
    np.testing.assert_array_equal(rotation.hadamard(g) * np.sqrt(g), scipy.linalg.hadamard(g))
    h = rotation.hadamard(g)
    np.testing.assert_allclose(h @ h.T, np.eye(g), atol=1e-14)
    np.testing.assert_allclose(h, h.T, atol=0)


def test_quaternion_multiplication_table():
    one, i, j, k = np.eye(4)
    np.testing.assert_array_equal(rotation.qmul(i, j), k)
    np.testing.assert_array_equal(rotation.qmul(j, k), i)
    np.testing.assert_array_equal(rotation.qmul(k, i), j)
    np.testing.assert_array_equal(rotation.qmul(j, i), -k)
    for u in (i, j, k):
        np.testing.assert_array_equal(rotation.qmul(u, u), -one)
    np.testing.assert_array_equal(rotation.qmul(rotation.qmul(i, j), k), -one)
    rng = np.random.default_rng(0)
    p, q = rng.standard_normal((2, 50, 4))
    np.testing.assert_allclose(np.linalg.norm(rotation.qmul(p, q), axis=-1),
                               np.linalg.norm(p, axis=-1) * np.linalg.norm(q, axis=-1), rtol=1e-13)


def left_matrix(q):
    """Matrix of v -> q v (written from the multiplication table, not from qmul)."""
    a, b, c, d = q
    return np.array([[a, -b, -c, -d], [b, a, -d, c], [c, d, a, -b], [d, -c, b, a]])


def right_matrix(q):
    """Matrix of v -> v q."""
    a, b, c, d = q
    return np.array([[a, -b, -c, -d], [b, a, d, -c], [c, -d, a, b], [d, c, -b, a]])


def test_so4_block_matches_matrix_form_and_is_special_orthogonal():
    rng = np.random.default_rng(1)
    so4 = unit_quats(rng, (32, 2))
    x = rng.standard_normal((5, 128))
    y = rotation.so4_forward(x, so4)
    for blk in range(32):
        ql, qr = so4[blk]
        conj = qr * np.array([1, -1, -1, -1])
        m = left_matrix(ql) @ right_matrix(conj)
        np.testing.assert_allclose(y[:, 4 * blk:4 * blk + 4], x[:, 4 * blk:4 * blk + 4] @ m.T, atol=1e-13)
        np.testing.assert_allclose(m @ m.T, np.eye(4), atol=1e-13)
        assert abs(np.linalg.det(m) - 1.0) < 1e-12
    np.testing.assert_allclose(rotation.so4_inverse(y, so4), x, atol=1e-13)


def test_single_quaternion_rotation_fixes_a_quarter_of_dimensions():
    # key design 2: q v conj(q) (one quaternion, SO(3)) leaves the real axis of every
    # 4-block unrotated, i.e. 25% of the dimensions; two independent quaternions do not.
    rng = np.random.default_rng(2)
    q = unit_quats(rng, (32,))
    same = np.stack([q, q], axis=1)
    basis = np.eye(128)
    y = rotation.so4_forward(basis, same)
    fixed = sum(np.allclose(y[c], basis[c], atol=1e-12) for c in range(128))
    assert fixed / 128 == FACTS["single_quaternion_unrotated_fraction"]["value"]
    y2 = rotation.so4_forward(basis, unit_quats(rng, (32, 2)))
    assert sum(np.allclose(y2[c], basis[c], atol=1e-6) for c in range(128)) == 0


@pytest.mark.parametrize("group,use_so4", [(32, False), (128, False), (128, True), (32, True)])
def test_rotation_orthogonal_and_inverse(group, use_so4):
    rng = np.random.default_rng(3)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    so4 = unit_quats(rng, (32, 2)) if use_so4 else None
    r = rotation.rotation_matrix(signs, group, so4)
    np.testing.assert_allclose(r @ r.T, np.eye(128), atol=1e-13)
    q, k = rng.standard_normal((2, 128))
    # key design 3: <Rq, Rk> = q^T k
    assert abs(rotation.rotate(q, signs, group, so4) @ rotation.rotate(k, signs, group, so4) - q @ k) < 1e-12
    x = rng.standard_normal((7, 128))
    np.testing.assert_allclose(rotation.unrotate(rotation.rotate(x, signs, group, so4), signs, group, so4),
                               x, atol=1e-13)


@pytest.mark.parametrize("group,use_so4", [(32, False), (128, True)])
def test_rotation_equals_independent_dense_construction(group, use_so4):
    # R = S_SO4 . blockdiag(H_g / sqrt(g)) . diag(s), built from scipy's Hadamard and the
    # 4x4 matrix forms; the oracle composes Hamilton products and reshapes instead.
    rng = np.random.default_rng(4)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    so4 = unit_quats(rng, (32, 2)) if use_so4 else None
    h = scipy.linalg.block_diag(*[scipy.linalg.hadamard(group) / np.sqrt(group)] * (128 // group))
    r = h @ np.diag(signs)
    if use_so4:
        blocks = [left_matrix(ql) @ right_matrix(qr * np.array([1, -1, -1, -1])) for ql, qr in so4]
        r = scipy.linalg.block_diag(*blocks) @ r
    np.testing.assert_allclose(rotation.rotation_matrix(signs, group, so4), r, atol=1e-14)


def test_operation_and_parameter_counts_on_page():
    # key design 2: a 128-point butterfly has log2(128) = 7 stages of 128 multiply-adds
    # (896), the SO(4) stage is 32 blocks of a 4x4 product (512), and the rotation keeps
    # 32 blocks x 2 quaternions x 4 = 256 parameters per head.
    d = 128
    assert d * int(np.log2(d)) == FACTS["wht_fma_d128"]["value"]
    assert (d // 4) * 16 == FACTS["so4_fma_d128"]["value"]
    assert FACTS["wht_fma_d128"]["value"] + FACTS["so4_fma_d128"]["value"] == FACTS["isoquant_total_fma"]["value"]
    assert round(d * d / FACTS["isoquant_total_fma"]["value"], 1) == FACTS["isoquant_fma_reduction"]["value"]
    so4 = np.zeros((d // 4, 2, 4))
    assert so4.size == FACTS["isoquant_params_per_head"]["value"]
    assert d * d // so4.size == FACTS["isoquant_param_reduction"]["value"]
    assert int(np.log2(FACTS["block_size"]["value"])) == FACTS["block_butterfly_stages"]["value"]

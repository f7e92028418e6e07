"""Pins for the oracle's attention, split/merge and rotated-domain rewrite.

* softmax attention vs scipy's softmax/logsumexp and torch's fp64 CPU
  scaled_dot_product_attention with grouped heads (fixes scale and the kv = h // G map);
* special cases: one token gives its value, a zero query gives the mean value;
* key-axis split + log-sum-exp merge equals the unsplit result for several split counts,
  including empty splits ("RoPE-Aware Bit Allocation ...", packed-cache details);
* computing straight from codes in the rotated domain with one inverse rotation equals
  dequantise-then-attend ("RotaryQuant ...", key design 3; "TurboQuant ...", 3.3).
"""

import math

import numpy as np
import pytest
import torch
from scipy import special

from oracle import attention, codebook, layout, quant


def unit_quats(rng, shape):
    q = rng.standard_normal(shape + (4,))
    return q / np.linalg.norm(q, axis=-1, keepdims=True)


def test_softmax_attend_matches_library():
    rng = np.random.default_rng(20)
    q = rng.standard_normal(128)
    k = rng.standard_normal((77, 128)) * 3
    v = rng.standard_normal((77, 128))
    scale = 128 ** -0.5
    o, lse = attention.softmax_attend(q, k, v, scale)
    s = scale * (k @ q)
    np.testing.assert_allclose(o, special.softmax(s) @ v, rtol=1e-13, atol=1e-14)
    assert abs(lse - special.logsumexp(s)) < 1e-12


def test_decode_matches_torch_sdpa_with_grouped_heads():
    rng = np.random.default_rng(21)
    b, hq, hkv, t = 2, 8, 2, 50
    q = rng.standard_normal((b, hq, 128))
    k = rng.standard_normal((b, hkv, t, 128))
    v = rng.standard_normal((b, hkv, t, 128))
    out, _ = attention.decode(q, k, v, np.full(b, t), 128 ** -0.5)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None], torch.from_numpy(k), torch.from_numpy(v), enable_gqa=True)[:, :, 0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-13)


def test_special_cases():
    rng = np.random.default_rng(22)
    v = rng.standard_normal((9, 128))
    o, _ = attention.softmax_attend(rng.standard_normal(128), rng.standard_normal((1, 128)), v[:1], 0.1)
    np.testing.assert_allclose(o, v[0], atol=1e-15)
    o, lse = attention.softmax_attend(np.zeros(128), rng.standard_normal((9, 128)), v, 0.1)
    np.testing.assert_allclose(o, v.mean(0), atol=1e-14)
    assert abs(lse - math.log(9)) < 1e-14
    o, lse = attention.softmax_attend(np.ones(128), np.zeros((0, 128)), np.zeros((0, 128)), 0.1)
    assert lse == -math.inf and not o.any()


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64, 100, 130])
def test_split_merge_equals_unsplit(n_splits):
    rng = np.random.default_rng(23)
    b, hq, hkv = 2, 4, 2
    lens = np.array([100, 37])
    q = rng.standard_normal((b, hq, 128))
    k = rng.standard_normal((b, hkv, 100, 128)) * 2
    v = rng.standard_normal((b, hkv, 100, 128))
    full, lse = attention.decode(q, k, v, lens, 0.09)
    po, pl = attention.decode_splits(q, k, v, lens, 0.09, n_splits)
    if n_splits > 37:
        assert np.isinf(pl[-1, 1]).all()          # some splits are empty
    out, lse2 = attention.merge(po, pl)
    np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


def test_two_stores_closed_form():
    # one token in each store, scores 0 and ln 3: weights 1/4 and 3/4, lse = ln 4
    scale = 0.5
    q = np.zeros((1, 1, 128))
    q[0, 0, 0] = 1.0
    ka = np.zeros((1, 1, 1, 128))
    kb = np.zeros((1, 1, 1, 128))
    kb[0, 0, 0, 0] = math.log(3.0) / scale
    rng = np.random.default_rng(30)
    va, vb = rng.standard_normal((1, 1, 1, 128)), rng.standard_normal((1, 1, 1, 128))
    out, lse = attention.decode_two_stores(q, ka, va, [1], kb, vb, [1], scale)
    np.testing.assert_allclose(out[0, 0], 0.25 * va[0, 0, 0] + 0.75 * vb[0, 0, 0], rtol=1e-14, atol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) < 1e-14


def test_two_stores_against_sdpa_and_invariants():
    rng = np.random.default_rng(31)
    b, hq, hkv = 2, 8, 2
    la, lb = np.array([40, 0]), np.array([9, 17])
    q = rng.standard_normal((b, hq, 128))
    ka, va = rng.standard_normal((b, hkv, 40, 128)) * 2, rng.standard_normal((b, hkv, 40, 128))
    kb, vb = rng.standard_normal((b, hkv, 17, 128)) * 2, rng.standard_normal((b, hkv, 17, 128))
    scale = 128 ** -0.5
    out, lse = attention.decode_two_stores(q, ka, va, la, kb, vb, lb, scale)
    # the library routine on the concatenated rows
    for i in range(b):
        k = np.concatenate([ka[i, :, :la[i]], kb[i, :, :lb[i]]], axis=1)
        v = np.concatenate([va[i, :, :la[i]], vb[i, :, :lb[i]]], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[i:i + 1])[:, :, None], torch.from_numpy(k[None]), torch.from_numpy(v[None]),
            scale=scale, enable_gqa=True)[0, :, 0]
        np.testing.assert_allclose(out[i], ref.numpy(), rtol=1e-12, atol=1e-13)
    # the stores' order does not matter; an empty store reduces to the other alone
    out2, lse2 = attention.decode_two_stores(q, kb, vb, lb, ka, va, la, scale)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)
    only_b, lse_b = attention.decode(q, kb, vb, lb, scale)
    np.testing.assert_allclose(out[1], only_b[1], rtol=1e-12, atol=1e-13)
    # and the union is the log-sum-exp merge of the two stores' section partials
    pa, la_s = attention.decode_splits(q, ka, va, la, scale, 3)
    pb, lb_s = attention.decode_splits(q, kb, vb, lb, scale, 2)
    m, ml = attention.merge(np.concatenate([pa, pb]), np.concatenate([la_s, lb_s]))
    np.testing.assert_allclose(m, out, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(ml, lse, rtol=1e-13)


def test_split_bounds_and_all_empty_merge():
    assert attention.split_bounds(10, 3) == [(0, 4), (4, 8), (8, 10)]
    assert attention.split_bounds(2, 4) == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert attention.split_bounds(0, 2) == [(0, 0), (0, 0)]
    out, lse = attention.merge(np.ones((3, 1, 2, 128)), np.full((3, 1, 2), -np.inf))
    assert not out.any() and np.isinf(lse).all()


@pytest.mark.parametrize("bits_k,bits_v,group,use_so4", [(3, 3, 32, False), (4, 3, 32, False),
                                                         (3, 3, 128, True), (4, 4, 128, False)])
def test_rotated_domain_equals_dequantise_then_attend(bits_k, bits_v, group, use_so4):
    rng = np.random.default_rng(24)
    b, hq, hkv, t = 2, 8, 2, 64
    signs = np.where(rng.random((hkv, 128)) < 0.5, -1.0, 1.0)
    so4 = unit_quats(rng, (hkv, 32, 2)) if use_so4 else None
    ck, mk = codebook.lloyd_max(bits_k, group)
    cv, mv = codebook.lloyd_max(bits_v, group)
    q = rng.standard_normal((b, hq, 128))
    kx = rng.standard_normal((b, hkv, t, 128))
    vx = rng.standard_normal((b, hkv, t, 128))
    kd = np.empty_like(kx)
    vd = np.empty_like(vx)
    kidx = np.empty(kx.shape, np.uint8)
    vidx = np.empty(vx.shape, np.uint8)
    kn = np.empty((b, hkv, t, 128 // group), np.float32)
    vn = np.empty_like(kn)
    for h in range(hkv):
        so = None if so4 is None else so4[h]
        kidx[:, h], kn[:, h], _ = quant.quantize(kx[:, h], signs[h], group, ck, mk, so)
        vidx[:, h], vn[:, h], _ = quant.quantize(vx[:, h], signs[h], group, cv, mv, so)
        kd[:, h] = quant.dequantize(kidx[:, h], kn[:, h], signs[h], group, ck, so)
        vd[:, h] = quant.dequantize(vidx[:, h], vn[:, h], signs[h], group, cv, so)
    lens = np.array([64, 41])
    ref, lse_ref = attention.decode(q, kd, vd, lens, 128 ** -0.5)
    out, lse = attention.decode_rotated_domain(q, kidx, kn, vidx, vn, lens, 128 ** -0.5, signs, group,
                                               ck, cv, so4)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-12)
    # the packed layout round-trips the exact codes used here
    np.testing.assert_array_equal(layout.unpack_values(layout.pack_values(vidx, bits_v), bits_v), vidx)
    np.testing.assert_array_equal(layout.unpack_keys(layout.pack_keys(kidx, bits_k), bits_k), kidx)


def test_quantised_attention_error_is_small_relative_to_exact():
    # reported, not a parity bar: 3-bit K/V attention stays close to unquantised attention
    rng = np.random.default_rng(25)
    signs = np.where(rng.random((1, 128)) < 0.5, -1.0, 1.0)
    c, m = codebook.lloyd_max(3, 32)
    q = rng.standard_normal((1, 4, 128))
    kx = rng.standard_normal((1, 1, 200, 128))
    vx = rng.standard_normal((1, 1, 200, 128))
    ki, kn, _ = quant.quantize(kx[:, 0], signs[0], 32, c, m)
    vi, vn, _ = quant.quantize(vx[:, 0], signs[0], 32, c, m)
    kd = quant.dequantize(ki, kn, signs[0], 32, c)[:, None]
    vd = quant.dequantize(vi, vn, signs[0], 32, c)[:, None]
    exact, _ = attention.decode(q, kx, vx, [200], 128 ** -0.5)
    approx, _ = attention.decode(q, kd, vd, [200], 128 ** -0.5)
    rel = np.linalg.norm(approx - exact) / np.linalg.norm(exact)
    assert rel < 0.35


@pytest.mark.parametrize("group,use_so4,hkv,g", [(32, False, 2, 4), (32, False, 1, 1), (128, True, 2, 4),
                                                 (128, False, 3, 2), (32, True, 2, 8)])
def test_rotate_heads_equals_dense_per_kv_head_rotation(group, use_so4, hkv, g):
    # Split partials are compared in the rotated domain of the query head's KV head
    # ("RotaryQuant ...", key design 3: one rotation per KV head, shared by its keys, values and
    # the queries that read it).  Each head's R is built here as a dense matrix from scipy's
    # Hadamard and the 4x4 matrix forms of the quaternion products, with the KV head of query
    # head h written out as h // g; a wrong head map, a dropped SO(4) stage or a transposed
    # R changes the result because every KV head has its own signs and quaternions.
    import scipy.linalg

    from test_oracle_rotation import left_matrix, right_matrix

    rng = np.random.default_rng(26)
    signs = np.where(rng.random((hkv, 128)) < 0.5, -1.0, 1.0)
    so4 = unit_quats(rng, (hkv, 32, 2)) if use_so4 else None
    hq = hkv * g
    x = rng.standard_normal((3, hq, 128))
    got = attention.rotate_heads(x, signs, group, so4, g)
    hblk = scipy.linalg.block_diag(*[scipy.linalg.hadamard(group) / np.sqrt(group)] * (128 // group))
    for h in range(hq):
        kv = h // g
        r = hblk @ np.diag(signs[kv])
        if use_so4:
            r = scipy.linalg.block_diag(*[left_matrix(ql) @ right_matrix(qr * np.array([1, -1, -1, -1]))
                                          for ql, qr in so4[kv]]) @ r
        np.testing.assert_allclose(got[:, h], x[:, h] @ r.T, atol=1e-13)

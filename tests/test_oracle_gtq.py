"""Pins of the Block-GTQ oracle ("RoPE-Aware Bit Allocation for KV-Cache Quantization":
block energies, the greedy integer allocation and its rate-law gain, one TQ-MSE encoder per
width) against brute force, closed forms and independent constructions."""

import itertools
import math

import numpy as np
import pytest
from scipy import special

from oracle import blockgtq as bg
from oracle import codebook


def test_energy_is_half_the_mean_block_second_moments():
    # two query heads per KV head; block i = coordinates (2i, 2i+1)
    rng = np.random.default_rng(0)
    q = rng.standard_normal((5, 4, 128))
    k = rng.standard_normal((5, 2, 128))
    s = bg.block_energies(q, k)
    for h in range(2):
        for i in (0, 7, 63):
            eq = np.mean([q[t, g, 2 * i] ** 2 + q[t, g, 2 * i + 1] ** 2 for t in range(5) for g in (2 * h, 2 * h + 1)])
            ek = np.mean([k[t, h, 2 * i] ** 2 + k[t, h, 2 * i + 1] ** 2 for t in range(5)])
            assert math.isclose(s[h, i], 0.5 * (eq + ek), rel_tol=1e-12)


def test_energy_hand_example():
    q = np.zeros((1, 1, 128))
    k = np.zeros((1, 1, 128))
    q[0, 0, 2:4] = [3.0, 4.0]   # block 1: ||q||^2 = 25
    k[0, 0, 3] = 2.0            # block 1: ||k||^2 = 4
    s = bg.block_energies(q, k)
    assert s[0, 1] == 14.5 and np.count_nonzero(s) == 1


@pytest.mark.parametrize("seed", range(6))
def test_greedy_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    L = 4 + seed % 3
    s = np.exp(rng.standard_normal(L) * 2)
    for b_min, b_max in ((1, 4), (0, 3), (2, 4)):
        for budget in range(L * b_min, L * b_max + 1):
            b = bg.allocate(s, budget, b_min, b_max)
            assert b.sum() == budget and b.min() >= b_min and b.max() <= b_max
            best, _ = bg.brute_force_min(s, budget, b_min, b_max)
            assert bg.objective(s, b) <= best * (1 + 1e-12)


def test_gain_is_the_closed_form():
    s = np.array([3.0, 0.5, 9.0])
    b = np.array([1, 2, 0])
    for i in range(3):
        up = b.copy()
        up[i] += 1
        assert math.isclose(bg.objective(s, b) - bg.objective(s, up), bg.rate_law_gain(s, b, i), rel_tol=1e-12)
        assert math.isclose(bg.rate_law_gain(s, b, i), 0.75 * s[i] * 4.0 ** -b[i], rel_tol=1e-15)


def test_greedy_favours_high_energy_blocks_and_breaks_ties_low():
    s = np.array([1.0, 64.0, 1.0, 1.0])
    # each extra bit divides a block's gain by 4: block 1 (64) takes 3 bits before any tie
    assert list(bg.allocate(s, 7, 1, 4)) == [1, 4, 1, 1]
    assert list(bg.allocate(s, 8, 1, 4)) == [2, 4, 1, 1]      # ties -> lowest index
    assert list(bg.allocate(np.ones(4), 6, 1, 4)) == [2, 2, 1, 1]
    with pytest.raises(ValueError):
        bg.allocate(s, 17, 1, 4)


def test_groups_partition_the_head_in_block_order():
    b = np.array([2, 1, 2, 4] + [1] * 60)
    gs = bg.groups(b)
    assert [w for w, _ in gs] == [1, 2, 4]
    assert list(gs[1][1]) == [0, 1, 4, 5] and list(gs[2][1]) == [6, 7]
    allc = np.concatenate([c for _, c in gs])
    assert sorted(allc) == list(range(128))


def gram_schmidt(a):
    # an independent construction: classical Gram-Schmidt on the columns, in fp64
    n = a.shape[0]
    q = np.zeros((n, n))
    for j in range(n):
        v = a[:, j].copy()
        for i in range(j):
            v -= (q[:, i] @ a[:, j]) * q[:, i]
        q[:, j] = v / np.linalg.norm(v)
    return q


@pytest.mark.parametrize("n", [2, 6, 30])
def test_rotation_is_the_unique_positive_qr_factor(n):
    g = np.random.default_rng(n).standard_normal((128, 128))
    qm = bg.rotation(g, n)
    assert np.allclose(qm.T @ qm, np.eye(n), atol=1e-12)
    assert np.allclose(qm, gram_schmidt(g[:n, :n]), atol=1e-10)
    r = qm.T @ g[:n, :n]
    assert np.all(np.diag(r) > 0) and np.allclose(np.tril(r, -1), 0, atol=1e-10)


@pytest.mark.parametrize("dim", [2, 3, 4, 6, 22, 128])
def test_one_bit_codebook_is_the_mean_absolute_coordinate(dim):
    # the 1-bit Lloyd-Max levels are +-E|t|: Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, m = codebook.lloyd_max(1, dim)
    ref = special.gamma(dim / 2) / (math.sqrt(math.pi) * special.gamma((dim + 1) / 2))
    assert math.isclose(c[1], ref, rel_tol=1e-10) and c[0] == -c[1] and m[0] == 0.0


def test_two_dimensional_law_is_the_arcsine_law():
    # a uniformly rotated unit vector in R^2 has coordinate cos(theta), theta uniform
    c, m = codebook.lloyd_max(2, 2)
    theta = np.random.default_rng(1).uniform(0, 2 * np.pi, 400000)
    t = np.cos(theta)
    cells = np.searchsorted(m, t)
    for k in range(4):
        assert abs(t[cells == k].mean() - c[k]) < 3e-3


def test_encode_decode_error_within_the_rate_law():
    rng = np.random.default_rng(2)
    s = np.exp(rng.standard_normal(64))
    b = bg.allocate(s, 192, 1, 4)
    gauss = rng.standard_normal((4, 128, 128))
    enc = bg.head_encoders(b, gauss)
    x = rng.standard_normal((400, 128))
    codes, norms, _ = bg.quantize_keys(x, enc)
    xr = bg.dequantize_keys(codes, norms, enc)
    for w, coords, qm, c, m in enc:
        n = len(coords)
        err = np.sum((x[:, coords] - xr[:, coords]) ** 2, axis=1) / np.sum(x[:, coords] ** 2, axis=1)
        # rotated unit coordinates follow the law: relative error = n * D1(w, n) on average
        assert abs(err.mean() - n * codebook.distortion(w, n)) < 0.1 * n * codebook.distortion(w, n) + 1e-3
    assert np.array_equal(bg.unpack_codes(bg.pack_codes(codes)), codes)


def test_codes_follow_the_compare_count_rule_and_zero_groups():
    rng = np.random.default_rng(3)
    b = np.array([1, 2, 3, 4] * 16)
    enc = bg.head_encoders(b, rng.standard_normal((4, 128, 128)))
    x = rng.standard_normal((3, 128))
    x[1, enc[0][1]] = 0.0                    # a zero group: norm 0, every coordinate 0
    codes, norms, ys = bg.quantize_keys(x, enc)
    assert norms[1, 0] == 0.0
    pos = 0
    for gi, (w, coords, qm, c, m) in enumerate(enc):
        n = len(coords)
        for t in range(3):
            for j in range(n):
                assert codes[t, pos + j] == np.searchsorted(m, ys[t, pos + j], side="left")
        pos += n


# ---- widths 5 to 8: byte containers ("RoPE-Aware Bit Allocation ...", packed-cache
# implementation details: low-bit groups in nibbles, high-bit groups in bytes)

def wide_allocation():
    # 4 high-energy blocks at 6 bits, two at 5, the rest at 3: budget 3.25 bits
    s = np.ones(64)
    s[[5, 9, 40, 63]] = 4.0 ** 3
    s[[7, 20]] = 4.0 ** 2
    b = bg.allocate(s, 208, 1, 8)
    assert sorted(set(b)) == [3, 5, 6]
    return b


def test_groups_and_allocation_up_to_eight_bits():
    b = wide_allocation()
    assert list(b[[5, 9, 40, 63]]) == [6] * 4 and list(b[[7, 20]]) == [5, 5]
    gs = bg.groups(b)
    assert [w for w, _ in gs] == [3, 5, 6]
    assert list(gs[1][1]) == [14, 15, 40, 41] and list(gs[2][1]) == [10, 11, 18, 19, 80, 81, 126, 127]
    # greedy = brute force with the wide range on a tiny head
    s = np.array([50.0, 1.0, 900.0])
    best, arg = bg.brute_force_min(s, 15, 1, 8)
    assert list(bg.allocate(s, 15, 1, 8)) == list(arg)


def _independent_record(codes, widths_by_position, record_bytes):
    """Writes one record position by position: nibbles while the width is at most 4 (two
    per byte, even position low), then one byte per position."""
    out = bytearray(record_bytes)
    byte, half = 0, 0
    for j, (c, w) in enumerate(zip(codes, widths_by_position)):
        if w <= 4:
            out[byte] |= int(c) << (4 * half)
            byte, half = (byte + half, 1 - half)
        else:
            out[byte] = int(c)
            byte += 1
    return list(out)


def test_byte_container_record_layout():
    rng = np.random.default_rng(11)
    b = wide_allocation()
    enc = bg.head_encoders(b, rng.standard_normal((8, 128, 128)))
    p = bg.nibble_positions(enc)
    assert p == 128 - 12 and bg.code_bytes(enc) == 80  # 58 nibble bytes + 12 bytes -> 80
    x = rng.standard_normal((6, 128))
    codes, norms, _ = bg.quantize_keys(x, enc)
    assert codes[:, p:].max() >= 16  # byte groups use their range
    packed = bg.pack_codes(codes, enc)
    widths = np.concatenate([np.full(len(coords), w) for w, coords, *_ in enc])
    for t in range(6):
        assert list(packed[t]) == _independent_record(codes[t], widths, 80)
    assert np.array_equal(bg.unpack_codes(packed, enc), codes)
    # a wider record for the whole cache keeps the layout and pads with zeros
    wide = bg.pack_codes(codes, enc, record_bytes=96)
    assert np.array_equal(wide[:, :80], packed) and not wide[:, 80:].any()
    # heads without wide groups keep the 64-byte nibble record
    enc4 = bg.head_encoders(np.array([1, 2, 3, 4] * 16), rng.standard_normal((8, 128, 128)))
    assert bg.code_bytes(enc4) == 64
    c4, _, _ = bg.quantize_keys(x, enc4)
    assert np.array_equal(bg.pack_codes(c4, enc4), bg.pack_codes(c4))


def test_wide_groups_encode_within_the_rate_law():
    rng = np.random.default_rng(12)
    enc = bg.head_encoders(wide_allocation(), rng.standard_normal((8, 128, 128)))
    x = rng.standard_normal((2000, 128))
    codes, norms, _ = bg.quantize_keys(x, enc)
    xr = bg.dequantize_keys(codes, norms, enc)
    for w, coords, qm, c, m in enc:
        n = len(coords)
        err = np.sum((x[:, coords] - xr[:, coords]) ** 2, axis=1) / np.sum(x[:, coords] ** 2, axis=1)
        d = n * codebook.distortion(w, n)
        assert abs(err.mean() - d) < 0.1 * d, (w, n, err.mean(), d)

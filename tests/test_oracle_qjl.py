"""Pins of the two-stage (MSE + QJL) key oracle ("TurboQuant ... MNN on phones", 2.4 and 3.2):
the Gaussian sign identity the estimator rests on, its unbiasedness and variance over random
projections, the MSE stage's inner-product shrink that the second stage removes, and the
sign packing.  Monte Carlo bounds are 5 standard errors."""

import math
import os

import numpy as np
import pytest

from oracle import blockgtq as bg
from oracle import codebook, qjl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_gaussian_sign_identity():
    # E[<s, q> sgn <s, r>] = sqrt(2/pi) <q, r> / |r| for s ~ N(0, I)
    rng = np.random.default_rng(0)
    d, n = 16, 400000
    q, r = rng.standard_normal(d), rng.standard_normal(d)
    s = rng.standard_normal((n, d))
    t = (s @ q) * np.sign(s @ r)
    want = math.sqrt(2 / math.pi) * (q @ r) / np.linalg.norm(r)
    se = math.sqrt((q @ q - (2 / math.pi) * (q @ r / np.linalg.norm(r)) ** 2) / n)
    assert abs(t.mean() - want) < 5 * se


def test_estimator_is_unbiased_with_the_closed_form_variance():
    rng = np.random.default_rng(1)
    d = m = 128
    q, r = rng.standard_normal(d), 0.3 * rng.standard_normal(d)
    n = 3000
    est = np.empty(n)
    for i in range(n):
        S = rng.standard_normal((m, d))
        signs, rn = qjl.encode_residual(r[None], S)
        est[i] = qjl.estimate(q, signs, rn, S)[0]
    var = qjl.estimate_variance(q, r, m)
    assert abs(est.mean() - q @ r) < 5 * math.sqrt(var / n)
    assert abs(est.var(ddof=1) / var - 1) < 5 * math.sqrt(2 / (n - 1))


def test_mse_stage_shrinks_and_two_stages_do_not():
    # 2.4: the MSE quantiser shrinks inner products; over uniformly random rotations
    # E<q, x_hat> = (1 - d D(b, d)) <q, x> exactly (centroid cells: E[c(Y) Y] = E[Y^2] - D).
    # At 1 bit that is about 2/pi.  Adding the QJL estimate of the residual removes it.
    rng = np.random.default_rng(2)
    d, n = 128, 1500
    x, q = rng.standard_normal(d), rng.standard_normal(d)
    x_dot_q = x @ q
    mse, two = np.empty(n), np.empty(n)
    for i in range(n):
        enc = qjl.mse_encoders(1, rng.standard_normal((4, d, d)))
        S = rng.standard_normal((d, d))
        codes, nu, signs, rn, xh = qjl.encode_keys(x[None], enc, S)
        mse[i] = xh[0] @ q
        two[i] = qjl.scores(q, xh, signs, rn, S)[0]
    shrink = 1 - d * codebook.distortion(1, d)
    assert abs(shrink - 2 / math.pi) < 0.01
    assert abs(mse.mean() - shrink * x_dot_q) < 5 * mse.std(ddof=1) / math.sqrt(n)
    assert abs(two.mean() - x_dot_q) < 5 * two.std(ddof=1) / math.sqrt(n)
    # and the shrink is a real bias at this sample size, not noise
    assert abs(mse.mean() - x_dot_q) > 10 * mse.std(ddof=1) / math.sqrt(n)


def test_encode_keys_stage_one_is_the_single_group_tq_mse():
    rng = np.random.default_rng(3)
    gauss = rng.standard_normal((4, 128, 128))
    for bits in (1, 2):
        enc = qjl.mse_encoders(bits, gauss)
        assert enc[0][0] == bits
        x = rng.standard_normal((5, 128))
        S = rng.standard_normal((128, 128))
        codes, nu, signs, rn, xh = qjl.encode_keys(x, enc, S)
        c2, n2, _ = bg.quantize_keys(x, enc)
        assert np.array_equal(codes, c2) and np.allclose(nu, n2[:, 0], rtol=0, atol=0)
        assert np.allclose(rn, np.linalg.norm(x - xh, axis=1), rtol=1e-12)
        assert np.array_equal(qjl.unpack_signs(signs), (x - xh) @ S.T >= 0)


def test_sign_packing_and_zero_residual():
    rng = np.random.default_rng(4)
    b = rng.random((7, 128)) < 0.5
    p = qjl.pack_signs(b)
    assert p.shape == (7, 16) and np.array_equal(qjl.unpack_signs(p), b)
    one = np.zeros(128, bool)
    one[9] = True  # bit 9 -> byte 1, bit 1
    assert list(qjl.pack_signs(one)[:3]) == [0, 2, 0]
    S = rng.standard_normal((128, 128))
    signs, rn = qjl.encode_residual(np.zeros((1, 128)), S)
    assert rn[0] == 0.0 and np.all(qjl.unpack_signs(signs))  # zero projections count as +
    assert qjl.estimate(rng.standard_normal(128), signs, rn, S)[0] == 0.0


def _bit_string_pack(codes, bits):
    """An independent writer of the stored layout: the key's codes as one Python integer,
    code i at bit bits * i, written out little-endian."""
    out = []
    for row in np.asarray(codes):
        word = 0
        for i, c in enumerate(row):
            word |= int(c) << (bits * i)
        out.append(list(word.to_bytes(16 * bits, "little")))
    return np.array(out, dtype=np.uint8)


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_stored_codes_layout(bits):
    # b - 1 bits per coordinate, bit-packed: 16, 32 or 48 bytes per key
    rng = np.random.default_rng(7 + bits)
    c = rng.integers(0, 1 << bits, (5, 128)).astype(np.uint8)
    p = qjl.pack_codes(c, bits)
    assert p.shape == (5, 16 * bits) == (5, qjl.code_bytes(bits))
    assert np.array_equal(p, _bit_string_pack(c, bits))
    assert np.array_equal(qjl.unpack_codes(p, bits), c)
    for i in (0, 13, 127):  # the top code at one position sets exactly its bits
        one = np.zeros((1, 128), np.uint8)
        one[0, i] = (1 << bits) - 1
        got = np.unpackbits(qjl.pack_codes(one, bits)[0], bitorder="little")
        assert list(np.flatnonzero(got)) == list(range(bits * i, bits * i + bits))
    with pytest.raises(AssertionError):
        qjl.pack_codes(np.full((1, 128), 1 << bits, np.uint8), bits)


def test_stored_codes_worked_examples():
    # at 1 bit: position 13 is byte 1, bit 5
    one = np.zeros((1, 128), np.uint8)
    one[0, 13] = 1
    assert list(qjl.pack_codes(one, 1)[0, :3]) == [0, 32, 0]
    # at 3 bits: the packed cache's hand-written three-byte words (tests/golden)
    n3 = 0
    for line in open(os.path.join(GOLDEN, "pack_layout_examples.txt")):
        f = line.split()
        if len(f) != 13 or f[0] != "word" or f[1] != "3":
            continue
        codes = np.zeros((1, 128), np.uint8)
        codes[0, :8] = [int(x, 16) for x in f[2:10]]
        assert list(qjl.pack_codes(codes, 3)[0, :3]) == [int(x, 16) for x in f[10:13]]
        n3 += 1
    assert n3 >= 5
    # at 2 bits: hand-written from the rule (code j of a byte at bits 2j .. 2j + 1)
    n2 = 0
    for line in open(os.path.join(GOLDEN, "qjl_code_layout.txt")):
        if line.startswith("#") or not line.strip():
            continue
        f = line.split()
        bits, codes_hex, bytes_hex = int(f[0]), f[1:9], f[9:]
        codes = np.zeros((1, 128), np.uint8)
        codes[0, :8] = [int(x, 16) for x in codes_hex]
        assert list(qjl.pack_codes(codes, bits)[0, :len(bytes_hex)]) == [int(x, 16) for x in bytes_hex]
        n2 += 1
    assert n2 >= 4


def test_one_bit_levels_split_into_midpoint_and_signs():
    # the decomposition the one-bit attention uses: <q, c[code]> = mid sum q + half <q, +-1>
    rng = np.random.default_rng(8)
    enc = qjl.mse_encoders(1, rng.standard_normal((4, 128, 128)))
    cent = np.asarray(enc[0][3], dtype=np.float64)
    assert cent.shape == (2,) and cent[0] < 0 < cent[1]
    x, q = rng.standard_normal((9, 128)), rng.standard_normal(128)
    codes, nu, _, _, xh = qjl.encode_keys(x, enc, rng.standard_normal((128, 128)))
    qt = enc[0][2].T @ q  # the rotated query, group order
    mid, half = cent.mean(), (cent[1] - cent[0]) / 2
    got = nu * (mid * qt.sum() + half * ((2.0 * codes - 1.0) @ qt))
    assert np.allclose(got, xh @ q, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [5, 6])
def test_attend_is_softmax_over_the_two_stage_scores(seed):
    rng = np.random.default_rng(seed)
    enc = qjl.mse_encoders(1, rng.standard_normal((4, 128, 128)))
    S = rng.standard_normal((128, 128))
    x, v, q = rng.standard_normal((40, 128)), rng.standard_normal((40, 128)), rng.standard_normal(128)
    _, _, signs, rn, xh = qjl.encode_keys(x, enc, S)
    s = 0.1 * qjl.scores(q, xh, signs, rn, S)
    w = np.exp(s - s.max())
    assert np.allclose(qjl.attend(q, xh, signs, rn, S, v, 0.1), (w / w.sum()) @ v, rtol=1e-12)

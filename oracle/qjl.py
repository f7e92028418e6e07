"""Two-stage keys: (b-1)-bit TQ-MSE plus a 1-bit QJL residual (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "TurboQuant ... MNN on phones", 2.4 (an MSE-optimal quantiser shrinks inner
products; for 1-2 bits the paper spends b - 1 bits on the MSE stage and 1 bit on QJL, a
random projection whose signs give an inner-product estimate that is unbiased in
expectation) and 3.2 (the two stages together make b bits; the projection matrix must be
stored).  The pages stop there; the readings below fill in the rest.

Readings: the MSE stage is the TQ-MSE encoder of the whole head as one group (norm ->
normalise -> uniformly random rotation -> Lloyd-Max search at b - 1 bits), i.e. a
Block-GTQ head with every block at width b - 1; the residual is r = x - x_hat in the
original coordinates; the projection S is an m x d matrix of independent N(0, 1) entries
drawn per KV head (m = d = 128), an input like the rotations; a key stores the m sign bits
of S r (a zero projection counts as +, bit i in byte i / 8 at bit i mod 8) and the scalar
|r|; the inner product with a query q is estimated as

    <q, x> ~ <q, x_hat> + sqrt(pi / 2) / m * |r| * sum_i (S q)_i sgn((S r)_i),

which is unbiased over S because, for s ~ N(0, I_d), E[<s, q> sgn <s, r>] equals
sqrt(2 / pi) <q, r> / |r| (the pair (<s, q>, <s, r>) is jointly Gaussian and
E[a sgn b] = sqrt(2 / pi) Cov(a, b) / sd(b) for centred jointly Gaussian a, b).
"""

import math

import numpy as np

from . import blockgtq

HEAD_DIM = 128


def mse_encoders(bits, gauss_by_width):
    """The MSE stage's encoder: one TQ-MSE group of all 128 coordinates at `bits` bits."""
    enc = blockgtq.head_encoders(np.full(blockgtq.BLOCKS, bits), gauss_by_width)
    assert len(enc) == 1 and list(enc[0][1]) == list(range(HEAD_DIM))
    return enc


def pack_signs(positive):
    """[..., m] booleans -> [..., m / 8] bytes, bit i in byte i // 8 at bit i % 8."""
    p = np.asarray(positive, dtype=bool)
    return np.packbits(p, axis=-1, bitorder="little")


def unpack_signs(packed, m=HEAD_DIM):
    return np.unpackbits(np.asarray(packed, dtype=np.uint8), axis=-1, bitorder="little", count=m).astype(bool)


def code_bytes(bits):
    """Stored bytes of one key's first-stage codes: b - 1 bits per coordinate, 128 of them."""
    return HEAD_DIM * bits // 8


def pack_codes(codes, bits):
    """The first stage's codes [T, 128] as stored, bit-packed at their own width ("TurboQuant
    ... MNN on phones", 3.2: the two stages take b bits per coordinate in total): code of
    position i at bit offset bits * i of the key's little-endian bit string, 16 * bits bytes.
    At 1 bit that is byte i // 8, bit i % 8 (the sign bits' order); at 2 bits four codes per
    byte; at 3 bits eight codes in three bytes, sum_j code_j << 3j, the packed cache's unit
    ("TurboQuant ...", 3.3)."""
    c = np.asarray(codes, dtype=np.uint8)
    assert bits in (1, 2, 3) and c.shape[-1] == HEAD_DIM and c.max(initial=0) < (1 << bits)
    planes = (c[..., :, None] >> np.arange(bits, dtype=np.uint8)) & 1  # [..., 128, bits], LSB first
    stream = planes.reshape(c.shape[:-1] + (HEAD_DIM * bits,)).astype(bool)
    return np.packbits(stream, axis=-1, bitorder="little")


def unpack_codes(packed, bits):
    p = np.asarray(packed, dtype=np.uint8)
    assert p.shape[-1] == code_bytes(bits)
    stream = np.unpackbits(p, axis=-1, bitorder="little", count=HEAD_DIM * bits)
    planes = stream.reshape(p.shape[:-1] + (HEAD_DIM, bits)).astype(np.uint8)
    return np.sum(planes << np.arange(bits, dtype=np.uint8), axis=-1).astype(np.uint8)


def encode_residual(r, S):
    """QJL of residuals r [T, d] with projection S [m, d] -> (sign bytes [T, m/8], |r| [T])."""
    r = np.asarray(r, dtype=np.float64)
    proj = r @ np.asarray(S, dtype=np.float64).T
    return pack_signs(proj >= 0.0), np.sqrt(np.sum(r * r, axis=1))


def estimate(q, signs, rnorm, S):
    """Unbiased estimate of <q, r> for every stored residual: q [d], signs [T, m/8],
    rnorm [T] -> [T]."""
    S = np.asarray(S, dtype=np.float64)
    m = S.shape[0]
    sq = S @ np.asarray(q, dtype=np.float64)
    pm = np.where(unpack_signs(signs, m), 1.0, -1.0)
    return math.sqrt(math.pi / 2.0) / m * np.asarray(rnorm, dtype=np.float64) * (pm @ sq)


def estimate_variance(q, r, m):
    """Variance over S of the estimate of <q, r> (closed form): each of the m terms
    |r| (s.q) sgn(s.r) has second moment |r|^2 |q|^2 and mean sqrt(2/pi) <q, r>."""
    q = np.asarray(q, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    rn = np.linalg.norm(r)
    return (math.pi / 2.0) / m * (rn * rn * (q @ q)) - (q @ r) ** 2 / m


def encode_keys(x, enc, S):
    """Two-stage encoding of keys x [T, 128]: (MSE codes [T, 128], MSE norm [T], sign bytes
    [T, m/8], |r| [T], x_hat [T, 128])."""
    x = np.asarray(x, dtype=np.float64)
    codes, norms, _ = blockgtq.quantize_keys(x, enc)
    xh = blockgtq.dequantize_keys(codes, norms, enc)
    signs, rn = encode_residual(x - xh, S)
    return codes, norms[:, 0], signs, rn, xh


def scores(q, xh, signs, rnorm, S):
    """Two-stage inner products of q [d] with every key: <q, x_hat> + the QJL estimate."""
    return np.asarray(xh, dtype=np.float64) @ np.asarray(q, dtype=np.float64) + estimate(q, signs, rnorm, S)


def attend(q, xh, signs, rnorm, S, v, scale):
    """Softmax attention of one query over two-stage keys and values v [T, d]."""
    s = scale * scores(q, xh, signs, rnorm, S)
    p = np.exp(s - np.max(s))
    return (p / p.sum()) @ np.asarray(v, dtype=np.float64)

"""Block-GTQ: RoPE-block bit allocation for the keys of a TurboQuant-MSE cache (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (aitrends.kr): the overview
(RoPE splits the head dimension into 2-D frequency blocks; the query-key logit is exactly a
sum of per-block dot products), the block energy score, the greedy integer allocation, the
grouping into one TQ-MSE encoder per bit width, and the packed-cache paragraphs (low-bit
groups in nibble containers, high-bit groups in bytes; the main benchmark evaluates keys
only, values kept in fp16).

* Energy of block i of KV head h: s_i = 1/2 (E_{t, g in G(h)} ||q_g,t^(i)||^2 +
  E_t ||k_h,t^(i)||^2), over a short calibration prefix; G(h) = the query heads reading h.
* Objective J(b) = sum_i s_i 4^(-b_i) (TurboQuant-MSE's rate law: error ~ 4^-b), subject to
  b_min <= b_i <= b_max and sum_i b_i = B.  Adding a bit to block i lowers J by
  Delta_i = (3/4) s_i 4^(-b_i); the greedy rule starts every block at b_min and gives the
  remaining B - L b_min bits one at a time to the block with the largest Delta_i.
* Blocks with the same width form one group, encoded by one TQ-MSE encoder (norm ->
  normalise -> rotate -> per-coordinate Lloyd-Max search at that width).

Readings (the pages leave these open): block i is coordinates (2i, 2i+1) (RoPE's 2-D
pairs); greedy ties go to the lowest block index; widths run from 1 to 8 bits, those up to
4 in nibble containers and 5 to 8 in byte containers; a group's coordinates are its blocks'
pairs in block order; its rotation is the orthogonal factor Q (with positive diagonal of R)
of the leading n x n part of a Gaussian matrix drawn per (KV head, width), n = the group's
dimension -- a uniformly random rotation, as the TurboQuant-MSE encoder assumes; the
codebook is the Lloyd-Max quantiser for a rotated unit vector's coordinate in n dimensions.
A token's key record holds the codes in group order (widths ascending, then the group's
rotated coordinate order): the P positions of nibble groups first, position j in byte j/2
(low nibble for even j), then the positions of byte groups, one byte each from byte P/2;
zero bytes pad it to the record size (64 bytes when no group is wider than 4 bits, else
the used bytes rounded up to 16, one size for a whole cache); and one fp32 norm per group.
"""

import heapq
import math

import numpy as np

from . import codebook

HEAD_DIM = 128
BLOCKS = HEAD_DIM // 2
MAX_WIDTH = 8
NIBBLE_MAX = 4  # widths above this take byte containers


def block_energies(q_cal, k_cal):
    """q_cal [N, Hq, 128], k_cal [N, Hkv, 128] -> s [Hkv, 64] (fp64)."""
    q = np.asarray(q_cal, dtype=np.float64)
    k = np.asarray(k_cal, dtype=np.float64)
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    qb = (q.reshape(q.shape[0], hq, BLOCKS, 2) ** 2).sum(-1)  # ||q^(i)||^2 per token, head
    kb = (k.reshape(k.shape[0], hkv, BLOCKS, 2) ** 2).sum(-1)
    s = np.zeros((hkv, BLOCKS))
    for h in range(hkv):
        s[h] = 0.5 * (qb[:, h * g:(h + 1) * g].mean(axis=(0, 1)) + kb[:, h].mean(axis=0))
    return s


def objective(s, b):
    return float(np.sum(np.asarray(s, np.float64) * 4.0 ** (-np.asarray(b, np.float64))))


def allocate(s, budget, b_min, b_max):
    """Greedy integer allocation: every block at b_min, then one bit at a time to the block
    with the largest marginal gain (3/4) s_i 4^-b_i among those below b_max."""
    s = np.asarray(s, dtype=np.float64)
    L = len(s)
    if not (L * b_min <= budget <= L * b_max):
        raise ValueError("budget outside [L b_min, L b_max]")
    b = np.full(L, b_min, dtype=np.int64)
    # a max-heap on the gain, ties to the lowest block index
    heap = [(-0.75 * s[i] * 4.0 ** (-b_min), i) for i in range(L) if b_min < b_max]
    heapq.heapify(heap)
    for _ in range(budget - L * b_min):
        _, i = heapq.heappop(heap)
        b[i] += 1
        if b[i] < b_max:
            heapq.heappush(heap, (-0.75 * s[i] * 4.0 ** (-float(b[i])), i))
    return b


def groups(b, b_min=1, b_max=MAX_WIDTH):
    """The groups of a head's allocation: [(width, coordinates)] for every width present,
    widths ascending, coordinates = the blocks' pairs in block order."""
    out = []
    for w in range(b_min, b_max + 1):
        blocks = [i for i in range(len(b)) if b[i] == w]
        if blocks:
            out.append((w, np.array([c for i in blocks for c in (2 * i, 2 * i + 1)], dtype=np.int64)))
    return out


def rotation(gauss, n):
    """The orthogonal factor of the leading n x n part of a Gaussian matrix (QR with the
    diagonal of R made positive, which makes the factor unique)."""
    a = np.asarray(gauss, dtype=np.float64)[:n, :n]
    qm, r = np.linalg.qr(a)
    return qm * np.sign(np.diag(r))[None, :]


def head_encoders(b, gauss_by_width):
    """[(width, coordinates, Q, centroids, boundaries)] for one KV head's groups.  A group
    vector u is rotated as y = Q^T u and restored as u = Q y."""
    enc = []
    for w, coords in groups(b):
        n = len(coords)
        qm = rotation(gauss_by_width[w - 1], n)
        c, m = codebook.lloyd_max(w, n)
        enc.append((w, coords, qm, c, m))
    return enc


def quantize_keys(x, enc):
    """x [T, 128] -> (codes [T, 128] in group order, norms [T, groups], y [T, 128] the
    rotated unit coordinates in group order, for boundary distances)."""
    x = np.asarray(x, dtype=np.float64)
    t = x.shape[0]
    codes = np.zeros((t, HEAD_DIM), dtype=np.uint8)
    norms = np.zeros((t, len(enc)))
    ys = np.zeros((t, HEAD_DIM))
    pos = 0
    for gi, (w, coords, qm, c, m) in enumerate(enc):
        n = len(coords)
        xg = x[:, coords]
        nu = np.sqrt(np.sum(xg * xg, axis=1))
        u = np.where(nu[:, None] > 0, xg / np.where(nu > 0, nu, 1.0)[:, None], 0.0)
        y = u @ qm  # y = Q^T u for every token (rows)
        codes[:, pos:pos + n] = np.sum(y[:, :, None] > m[None, None, :], axis=2)  # compare-count
        norms[:, gi] = nu
        ys[:, pos:pos + n] = y
        pos += n
    return codes, norms, ys


def dequantize_keys(codes, norms, enc):
    """Inverse: [T, 128] in the original coordinate order."""
    codes = np.asarray(codes)
    t = codes.shape[0]
    out = np.zeros((t, HEAD_DIM))
    pos = 0
    for gi, (w, coords, qm, c, m) in enumerate(enc):
        n = len(coords)
        y = c[codes[:, pos:pos + n].astype(np.int64)]
        out[:, coords] = (y @ qm.T) * norms[:, gi:gi + 1]  # x = nu Q y
        pos += n
    return out


def nibble_positions(enc):
    """P: the group-order positions held in nibbles (the groups of width <= 4 come first)."""
    return sum(len(coords) for w, coords, *_ in enc if w <= NIBBLE_MAX)


def code_bytes(enc):
    """Code bytes one record of this head needs: 64 when every group fits a nibble, else the
    P / 2 nibble bytes plus one byte per wider position, rounded up to 16."""
    p = nibble_positions(enc)
    if p == HEAD_DIM:
        return HEAD_DIM // 2
    return -(-(p // 2 + HEAD_DIM - p) // 16) * 16


def pack_codes(codes, enc=None, record_bytes=None):
    """[T, 128] codes in group order -> [T, record_bytes] bytes.  Without enc every position
    is a nibble (64 bytes: code j in byte j // 2, low nibble for even j); with enc the
    positions past the nibble groups take one byte each from byte P / 2, and zero bytes pad
    the record to record_bytes (default: code_bytes(enc))."""
    codes = np.asarray(codes, dtype=np.uint8)
    p = HEAD_DIM if enc is None else nibble_positions(enc)
    r = (HEAD_DIM // 2 if enc is None else code_bytes(enc)) if record_bytes is None else record_bytes
    assert p % 2 == 0 and r >= p // 2 + HEAD_DIM - p
    assert np.all(codes[:, :p] < 16)
    out = np.zeros((codes.shape[0], r), dtype=np.uint8)
    out[:, :p // 2] = (codes[:, 0:p:2] & 0xF) | ((codes[:, 1:p:2] & 0xF) << 4)
    out[:, p // 2:p // 2 + HEAD_DIM - p] = codes[:, p:]
    return out


def unpack_codes(packed, enc=None):
    p_ = np.asarray(packed, dtype=np.uint8)
    p = HEAD_DIM if enc is None else nibble_positions(enc)
    out = np.zeros((p_.shape[0], HEAD_DIM), dtype=np.uint8)
    out[:, 0:p:2] = p_[:, :p // 2] & 0xF
    out[:, 1:p:2] = p_[:, :p // 2] >> 4
    out[:, p:] = p_[:, p // 2:p // 2 + HEAD_DIM - p]
    return out


def rate_law_gain(s, b, i):
    """J(b) - J(b + e_i), the closed form (3/4) s_i 4^-b_i."""
    return 0.75 * float(s[i]) * 4.0 ** (-float(b[i]))


def decode(q, keys_dequantized, v, seq_lens, scale):
    """Attention of q[B, Hq, 128] over dequantised keys and unquantised values."""
    from . import attention
    return attention.decode(q, keys_dequantized, v, seq_lens, scale)


def brute_force_min(s, budget, b_min, b_max):
    """Minimum of J over every integer allocation (tiny L only)."""
    L = len(s)
    best, arg = math.inf, None
    for b in np.ndindex(*([b_max - b_min + 1] * L)):
        bb = np.array(b) + b_min
        if bb.sum() == budget:
            j = objective(s, bb)
            if j < best:
                best, arg = j, bb
    return best, arg

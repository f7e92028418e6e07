"""Plain softmax decode attention over explicitly dequantised K/V (oracle, fp64).

Sources:
* dequantise-then-attend is the "reconstruct then compute" path the pages replace
  ("RotaryQuant ... Fused Compressed-Space Attention", research background); it is the
  plain definition the compressed-domain kernels must reproduce, because
  <Rq, Rk> = q^T k and sum_j a_j R v_j = R o ("RotaryQuant ...", key design 3;
  "TurboQuant ... MNN on phones", 3.3).
* long contexts are split along the key axis and the sections merged by log-sum-exp
  ("RoPE-Aware Bit Allocation for KV-Cache Quantization", packed-cache implementation
  details).

Readings: softmax scale is an explicit argument (1/sqrt(128) for every workload here);
query head h reads KV head h // G with G = H_q / H_kv (contiguous groups); split s of a
length-T row covers tokens [s*C, min(T, (s+1)*C)) with C = ceil(T / S); an empty split
has lse = -inf and a zero partial; a row with no tokens yields out = 0 and lse = -inf.
"""

import math

import numpy as np

from . import rotation


def softmax_attend(q, k, v, scale):
    """One query row q[d] against k[T, d], v[T, d]: returns (o[d], lse) in fp64.

    s_j = scale * <q, k_j>; a = exp(s - max) / sum; o = sum_j a_j v_j; lse = ln sum_j e^{s_j}.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if k.shape[0] == 0:
        return np.zeros(q.shape[-1]), -math.inf
    s = scale * (k @ q)
    mx = np.max(s)
    e = np.exp(s - mx)
    z = np.sum(e)
    return (e @ v) / z, mx + math.log(z)


def decode(q, k, v, seq_lens, scale):
    """q[B, Hq, d], k/v[B, Hkv, T, d] (already dequantised) -> (out[B, Hq, d], lse[B, Hq])."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        t = int(seq_lens[b])
        for h in range(hq):
            out[b, h], lse[b, h] = softmax_attend(q[b, h], k[b, h // g, :t], v[b, h // g, :t], scale)
    return out, lse


def decode_two_stores(q, k_a, v_a, lens_a, k_b, v_b, lens_b, scale):
    """Attention of every query row over the union of two token stores of its row.

    Store a holds the quantised tokens (already dequantised), store b the unquantised ones:
    the prefill kept in fp16 while decode-phase tokens are quantised ("RotaryQuant ...",
    method overview), or a window of recent tokens ("RoPE-Aware Bit Allocation ...", results:
    the recent-token buffer).  Softmax attention is a sum over the row's tokens, so the union
    is their concatenation: k_a[b, kv, :lens_a[b]] followed by k_b[b, kv, :lens_b[b]].
    Returns (out[B, Hq, d], lse[B, Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    g = hq // k_a.shape[1]
    out = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    for b in range(bsz):
        la, lb = int(lens_a[b]), int(lens_b[b])
        for h in range(hq):
            kv = h // g
            k = np.concatenate([np.asarray(k_a[b, kv, :la], np.float64), np.asarray(k_b[b, kv, :lb], np.float64)])
            v = np.concatenate([np.asarray(v_a[b, kv, :la], np.float64), np.asarray(v_b[b, kv, :lb], np.float64)])
            out[b, h], lse[b, h] = softmax_attend(q[b, h], k, v, scale)
    return out, lse


def split_bounds(t, n_splits):
    """Token ranges of the key-axis splits: chunk C = ceil(t / S)."""
    c = -(-t // n_splits) if t > 0 else 0
    return [(min(t, s * c), min(t, (s + 1) * c)) for s in range(n_splits)]


def decode_splits(q, k, v, seq_lens, scale, n_splits):
    """Per-split partial outputs (original domain) and lse: o[S, B, Hq, d], lse[S, B, Hq]."""
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    po = np.zeros((n_splits, bsz, hq, d))
    pl = np.full((n_splits, bsz, hq), -math.inf)
    for b in range(bsz):
        for s, (lo, hi) in enumerate(split_bounds(int(seq_lens[b]), n_splits)):
            for h in range(hq):
                po[s, b, h], pl[s, b, h] = softmax_attend(q[b, h], k[b, h // g, lo:hi],
                                                          v[b, h // g, lo:hi], scale)
    return po, pl


def merge(part_o, part_lse):
    """Log-sum-exp merge over the leading split axis: returns (out, lse)."""
    part_o = np.asarray(part_o, dtype=np.float64)
    part_lse = np.asarray(part_lse, dtype=np.float64)
    mx = np.max(part_lse, axis=0)
    finite = np.isfinite(mx)
    mx_safe = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(part_lse), np.exp(part_lse - mx_safe), 0.0)
    z = np.sum(w, axis=0)
    zs = np.where(z > 0, z, 1.0)
    out = np.sum(w[..., None] * part_o, axis=0) / zs[..., None]
    lse = np.where(z > 0, mx_safe + np.log(zs), -math.inf)
    return out, lse


def rotate_heads(x, signs, group, so4, g):
    """Rotate x[B, Hq, d] (query heads) with the rotation of KV head h // g."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    for h in range(x.shape[1]):
        kv = h // g
        out[:, h] = rotation.rotate(x[:, h], signs[kv], group, None if so4 is None else so4[kv])
    return out


def decode_rotated_domain(q, k_idx, k_norms, v_idx, v_norms, seq_lens, scale, signs, group,
                          k_centroids, v_centroids, so4=None):
    """Self-check of the compressed-domain rewrite, straight from codes and norms.

    q_rot = R q once per head; s_j = scale * sum_groups n_j,grp <q_rot_grp, c[idx_j,grp]>;
    o_rot = sum_j a_j n_j,grp c[idx_j]; o = R^T o_rot.  Equal to ``decode`` on the
    dequantised cache up to rounding ("RotaryQuant ...", key design 3).
    """
    q = np.asarray(q, dtype=np.float64)
    bsz, hq, d = q.shape
    hkv = k_idx.shape[1]
    g = hq // hkv
    ng = d // group
    out = np.zeros((bsz, hq, d))
    lse = np.zeros((bsz, hq))
    kc = np.asarray(k_centroids, dtype=np.float64)
    vc = np.asarray(v_centroids, dtype=np.float64)
    for b in range(bsz):
        t = int(seq_lens[b])
        for h in range(hq):
            kv = h // g
            so = None if so4 is None else so4[kv]
            qr = rotation.rotate(q[b, h], signs[kv], group, so)
            kk = (kc[k_idx[b, kv, :t]].reshape(t, ng, group) *
                  np.asarray(k_norms[b, kv, :t], dtype=np.float64)[..., None]).reshape(t, d)
            vv = (vc[v_idx[b, kv, :t]].reshape(t, ng, group) *
                  np.asarray(v_norms[b, kv, :t], dtype=np.float64)[..., None]).reshape(t, d)
            orot, lse[b, h] = softmax_attend(qr, kk, vv, scale)
            out[b, h] = rotation.unrotate(orot, signs[kv], group, so)
    return out, lse

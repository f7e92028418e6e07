"""Test-side helpers: oracle-quantised caches in the library layout and parity metrics.

Everything here calls only ``oracle`` and ``workloads``; nothing is derived from the HIP
path.  Tolerances (from the parity bar): codes bit-exact except coordinates within 1e-6
of a decision boundary (on the oracle's fp64 value) and at most 1e-5 of all coordinates;
norms within 1e-6 relative; attention outputs within 2e-3 max relative error per row.
"""

import numpy as np

from oracle import attention, codebook, layout, quant, rotation

CODE_BOUNDARY_EPS = 1e-6
CODE_FLIP_FRACTION = 1e-5
NORM_RTOL = 1e-6
OUT_RTOL = 2e-3


def round_up(x, m):
    return (x + m - 1) // m * m


def oracle_quantize(w, inp, role):
    """Oracle codes/norms/boundary distances for the workload's K or V: per (b, kv) head."""
    x = inp["k"] if role == "k" else inp["v"]
    bits = w.bits_k if role == "k" else w.bits_v
    c, m = codebook.lloyd_max(bits, w.group)
    bsz, hkv, t, d = x.shape
    idx = np.zeros((bsz, hkv, t, d), np.uint8)
    norms = np.zeros((bsz, hkv, t, d // w.group), np.float32)
    dist = np.zeros((bsz, hkv, t, d))
    for kv in range(hkv):
        so = None if inp["so4"] is None else inp["so4"][kv]
        i, n, y = quant.quantize(x[:, kv].astype(np.float64), inp["signs"][kv], w.group, c, m, so)
        idx[:, kv], norms[:, kv], dist[:, kv] = i, n, quant.boundary_distance(y, m)
    return {"idx": idx, "norms": norms, "dist": dist, "bits": bits, "centroids": c}


def pad_tokens(a, cap):
    out = np.zeros(a.shape[:2] + (cap,) + a.shape[3:], a.dtype)
    out[:, :, :a.shape[2]] = a
    return out


def pack(oq, cap, role):
    idx = pad_tokens(oq["idx"], cap)
    codes = layout.pack_keys(idx, oq["bits"]) if role == "k" else layout.pack_values(idx, oq["bits"])
    return codes, layout.pack_norms(pad_tokens(oq["norms"], cap))


def unpack(codes, norms, bits, role):
    idx = layout.unpack_keys(codes, bits) if role == "k" else layout.unpack_values(codes, bits)
    return idx, layout.unpack_norms(norms)


def dequantized(w, inp, oq):
    out = np.zeros(oq["idx"].shape)
    for kv in range(oq["idx"].shape[1]):
        so = None if inp["so4"] is None else inp["so4"][kv]
        out[:, kv] = quant.dequantize(oq["idx"][:, kv], oq["norms"][:, kv], inp["signs"][kv], w.group,
                                      oq["centroids"], so)
    return out


def check_codes(got_idx, got_norms, oq, t, rate_bar=True):
    """Assert the code and norm bar; returns the number of excused near-boundary flips.
    rate_bar=False leaves the flip rate to the caller (which pools it over several cases)."""
    ref, dist = oq["idx"], oq["dist"]
    g = got_idx[:, :, :t]
    diff = g != ref
    flips = int(diff.sum())
    assert np.all(dist[diff] < CODE_BOUNDARY_EPS), "code mismatch away from a boundary"
    if rate_bar:
        assert flips <= CODE_FLIP_FRACTION * ref.size + 0, "too many near-boundary flips: %d" % flips
    n_ref = oq["norms"].astype(np.float64)
    n_got = got_norms[:, :, :t].astype(np.float64)
    zero = n_ref == 0
    assert np.all(n_got[zero] == 0)
    rel = np.abs(n_got[~zero] - n_ref[~zero]) / n_ref[~zero]
    assert rel.max(initial=0.0) <= NORM_RTOL, "norm rel err %g" % rel.max()
    return flips


def row_rel_err(got, ref):
    """max_i |got - ref| / max_i |ref| per row (rows with ref == 0 use absolute error)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def oracle_decode(w, inp, kd, vd, seq_lens, n_splits=1):
    q = inp["q"].astype(np.float64)
    if n_splits == 1:
        return attention.decode(q, kd, vd, seq_lens, w.scale)
    po, pl = attention.decode_splits(q, kd, vd, seq_lens, w.scale, n_splits)
    # the library's partials live in the rotated domain of the head's KV rotation
    g = w.group_size
    rot = np.empty_like(po)
    for s in range(n_splits):
        rot[s] = attention.rotate_heads(po[s], inp["signs"], w.group, inp["so4"], g)
    return rot, pl

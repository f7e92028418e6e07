"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Sizes are small enough for the oracle yet span several 32-token tiles and a ragged tail;
every workload family is covered (fp32 tiny, 4B-style GQA, TQ4 keys / TQ3 values, G=8
with log-normal channel scales, IsoQuant whole-head rotation with SO(4) blocks).
Decode parity feeds the same oracle-packed cache to both sides.
"""

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import (OUT_RTOL, check_codes, dequantized, oracle_decode, oracle_quantize, pack, round_up,
                     row_rel_err, unpack)
from oracle import attention, rotation

pytestmark = pytest.mark.gpu

CASES = {
    "tiny": dict(seq_len=256, batch=1),
    "gqa8k": dict(seq_len=300, batch=1),
    "batched": dict(seq_len=100, batch=2),
    "long128k": dict(seq_len=200, batch=1),
    "isoquant32k": dict(seq_len=96, batch=2),
}


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()  # raises if the native library is missing


def setup(name, seed=0, **over):
    kw = dict(CASES[name])
    kw.update(over)
    w = workloads.WORKLOADS[name].with_len(kw["seq_len"], batch=kw["batch"])
    inp = workloads.generate(w, seed)
    print("case", name, "seed", seed, "shape", (w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len), flush=True)
    return w, inp


def device_rotation(w, inp):
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).cuda()
    return tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, so4)


def empty_caches(w, cap):
    k = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS)
    v = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES)
    return k, v


def oracle_caches(w, inp, cap):
    """Oracle quantisation packed into the library layout, as device caches."""
    oqk, oqv = oracle_quantize(w, inp, "k"), oracle_quantize(w, inp, "v")
    kc, kn = pack(oqk, cap, "k")
    vc, vn = pack(oqv, cap, "v")
    k = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS,
                       codes=torch.from_numpy(kc).cuda(), norms=torch.from_numpy(kn).cuda())
    v = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES,
                       codes=torch.from_numpy(vc).cuda(), norms=torch.from_numpy(vn).cuda())
    return k, v, oqk, oqv


def download(cache, role):
    idx, n = unpack(cache.codes.cpu().numpy(), cache.norms.cpu().numpy(), cache.bits, role)
    return idx, n


@pytest.mark.parametrize("name", list(CASES))
def test_append_matches_oracle(name):
    w, inp = setup(name)
    t = w.seq_len
    cap = round_up(t, 32) + 32
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, cap)
    tq.quantize_append(rot, k, torch.from_numpy(inp["k"]).cuda())
    tq.quantize_append(rot, v, torch.from_numpy(inp["v"]).cuda())
    torch.cuda.synchronize()
    total_flips = 0
    for role, cache in (("k", k), ("v", v)):
        oq = oracle_quantize(w, inp, role)
        idx, n = download(cache, role)
        total_flips += check_codes(idx, n, oq, t)
        assert not idx[:, :, t:].any() and not n[:, :, t:].any(), "slots past the appended range were written"
    print("near-boundary flips", total_flips, flush=True)


def test_append_incremental_and_device_positions():
    # prefill part of each row, then single-token steps, then a chunk at per-row device
    # positions: partial 32-token tiles are read-modify-written and must keep neighbours
    w, inp = setup("batched", seq_len=90, batch=2)
    t = w.seq_len
    cap = 128
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, cap)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    p1 = 37
    for cache, x in ((k, kx), (v, vx)):
        tq.quantize_append(rot, cache, x[:, :, :p1].contiguous(), pos0=0)
        for s in range(p1, 45):
            tq.quantize_append(rot, cache, x[:, :, s:s + 1].contiguous(), pos0=s)
        pos = torch.tensor([45, 45], dtype=torch.int32, device="cuda")
        tq.quantize_append(rot, cache, x[:, :, 45:t].contiguous(), pos=pos)
    torch.cuda.synchronize()
    for role, cache in (("k", k), ("v", v)):
        idx, n = download(cache, role)
        check_codes(idx, n, oracle_quantize(w, inp, role), t)
        assert not idx[:, :, t:].any()


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("name", ["gqa8k", "batched", "isoquant32k"])
def test_append_whole_tiles_between_partial_edges(name, fused):
    # a chunk that starts and ends inside a 32-token tile: the whole tiles between take the
    # matrix-core append (fp16 vectors, one start position for every row), the partial
    # tiles at both ends the tile kernel, which must keep the earlier tokens of the first
    w, inp = setup(name, seq_len=190, batch=2)
    t, p0 = w.seq_len, 7
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, 224)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    for lo, hi in ((0, p0), (p0, t)):
        xs, ys = kx[:, :, lo:hi].contiguous(), vx[:, :, lo:hi].contiguous()
        if fused:
            tq.quantize_append_kv(rot, k, v, xs, ys, pos0=lo)
        else:
            tq.quantize_append(rot, k, xs, pos0=lo)
            tq.quantize_append(rot, v, ys, pos0=lo)
    torch.cuda.synchronize()
    for role, cache in (("k", k), ("v", v)):
        idx, n = download(cache, role)
        check_codes(idx, n, oracle_quantize(w, inp, role), t)
        assert not idx[:, :, t:].any() and not n[:, :, t:].any()


@pytest.mark.parametrize("name", ["batched", "isoquant32k", "tiny"])
def test_fused_append_equals_separate_calls(name):
    # multi-token appends in one launch give the two separate calls' bytes exactly: a
    # prefill into a fresh cache, then a partial-tile chunk at per-row device positions
    w, inp = setup(name, seed=7, seq_len=70, batch=2)
    cap = 128
    rot = device_rotation(w, inp)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    k1, v1 = empty_caches(w, cap)
    k2, v2 = empty_caches(w, cap)
    p1 = 37
    tq.quantize_append(rot, k1, kx[:, :, :p1].contiguous())
    tq.quantize_append(rot, v1, vx[:, :, :p1].contiguous())
    tq.quantize_append_kv(rot, k2, v2, kx[:, :, :p1].contiguous(), vx[:, :, :p1].contiguous())
    pos = torch.full((w.batch,), p1, dtype=torch.int32, device="cuda")
    xs, ys = kx[:, :, p1:].contiguous(), vx[:, :, p1:].contiguous()
    tq.quantize_append(rot, k1, xs, pos=pos)
    tq.quantize_append(rot, v1, ys, pos=pos)
    tq.quantize_append_kv(rot, k2, v2, xs, ys, pos=pos)
    torch.cuda.synchronize()
    for a, b in ((k1, k2), (v1, v2)):
        assert torch.equal(a.codes, b.codes) and torch.equal(a.norms, b.norms)


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("name", list(CASES))
def test_append_decode_equals_separate_calls(name, schedule):
    # one call that appends each row's new token and decodes over rows ending at it gives
    # the cache bytes and the outputs of the append call followed by the decode call: at a
    # host position and at per-row device positions (one overwriting an earlier slot), whole
    # and split, where the section holding the new token is the last one, an inner one
    # (short sections, empty ones after it) or the only one
    w, inp = setup(name, seed=9, seq_len=80, batch=2)
    cap = 96
    rot = device_rotation(w, inp)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    q = torch.from_numpy(inp["q"]).cuda()
    p = 61
    xs, ys = kx[:, :, p:p + 1].contiguous(), vx[:, :, p:p + 1].contiguous()
    for device_pos in (False, True):
        for n_splits in (1, 4, 40):
            k1, v1 = empty_caches(w, cap)
            k2, v2 = empty_caches(w, cap)
            for k, v in ((k1, v1), (k2, v2)):
                tq.quantize_append_kv(rot, k, v, kx[:, :, :p].contiguous(), vx[:, :, :p].contiguous())
            if device_pos:
                pos = torch.tensor([p, p - 5], dtype=torch.int32, device="cuda")
                kw = dict(pos=pos, max_pos=p)
                tq.quantize_append_kv(rot, k1, v1, xs, ys, **kw)
                r1 = tq.decode_attention(rot, k1, v1, q, seq_lens=pos + 1, max_len=p + 1, n_splits=n_splits,
                                         schedule=schedule)
            else:
                kw = dict(pos0=p)
                tq.quantize_append_kv(rot, k1, v1, xs, ys, **kw)
                r1 = tq.decode_attention(rot, k1, v1, q, max_len=p + 1, n_splits=n_splits, schedule=schedule)
            r2 = tq.append_decode_attention(rot, k2, v2, xs, ys, q, n_splits=n_splits, schedule=schedule, **kw)
            torch.cuda.synchronize()
            print("positions %s, splits %d" % ("device" if device_pos else "host", n_splits), flush=True)
            for a, b in ((k1, k2), (v1, v2)):
                assert torch.equal(a.codes, b.codes) and torch.equal(a.norms, b.norms)
            for a, b in zip(r1, r2):
                assert torch.equal(a, b)


DENSE_RTOL = 1e-4  # fp32 scores and sums over unquantised inputs


@pytest.mark.parametrize("n_splits", [1, 3, 40])
@pytest.mark.parametrize("name", list(CASES))
def test_dense_sections_match_oracle(name, n_splits):
    # unquantised K/V (the workload's dtype): section partials in the rotated domain and their
    # merge, ragged rows including an empty one
    w, inp = setup(name, seed=11, seq_len=150, batch=3)
    rot = device_rotation(w, inp)
    k, v = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    q = torch.from_numpy(inp["q"]).cuda()
    lens = np.array([150, 0, 67], dtype=np.int32)
    po, pl = tq.dense_attention(rot, k, v, q, seq_lens=torch.from_numpy(lens).cuda(), max_len=150,
                                n_splits=n_splits)
    out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    kd, vd = inp["k"].astype(np.float64), inp["v"].astype(np.float64)
    ref, ref_lse = oracle_decode(w, inp, kd, vd, lens)
    err = row_rel_err(out.cpu().numpy(), ref)
    print("dense: max row rel err %.3e (splits %d)" % (err.max(), n_splits), flush=True)
    assert err.max() <= DENSE_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)
    if n_splits > 1:
        ref_po, ref_pl = oracle_decode(w, inp, kd, vd, lens, n_splits)
        assert row_rel_err(po.cpu().numpy(), ref_po).max() <= DENSE_RTOL
        np.testing.assert_allclose(pl.cpu().numpy(), ref_pl, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("kv_dtype,q_dtype,n_q_heads", [(np.float16, np.float32, 32), (np.float16, np.float16, 64),
                                                     (np.float32, np.float16, 64)])
def test_dense_query_dtypes_and_head_slices(kv_dtype, q_dtype, n_q_heads):
    # both query dtypes against fp16 and fp32 rows, and 16 query heads per KV head (two
    # workgroup slices of 8), with ragged rows and an empty one
    from dataclasses import replace
    w, inp = setup("long128k", seed=13, seq_len=150, batch=3)
    w = replace(w, n_q_heads=n_q_heads)
    rng = np.random.default_rng(13)
    q32 = (rng.standard_normal((w.batch, n_q_heads, 128)) * 0.5).astype(np.float16).astype(np.float32)
    inp = dict(inp, q=q32.astype(q_dtype))
    rot = device_rotation(w, inp)
    kx = inp["k"].astype(kv_dtype)
    vx = inp["v"].astype(kv_dtype)
    lens = np.array([150, 0, 67], dtype=np.int32)
    po, pl = tq.dense_attention(rot, torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda(),
                                torch.from_numpy(inp["q"]).cuda(), seq_lens=torch.from_numpy(lens).cuda(),
                                max_len=150, n_splits=3)
    out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(w, inp, kx.astype(np.float64), vx.astype(np.float64), lens)
    err = row_rel_err(out.cpu().numpy(), ref)
    print("dense %s K/V, %s q, %d heads: max row rel err %.3e" % (np.dtype(kv_dtype).name, np.dtype(q_dtype).name,
                                                                  n_q_heads, err.max()), flush=True)
    assert err.max() <= DENSE_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name", list(CASES))
def test_packed_prefix_with_unquantised_tail(name):
    # a row is a packed prefix plus an unquantised tail (recent tokens, or an fp16 prefill):
    # packed sections and dense sections share one partial buffer and one merge
    w, inp = setup(name, seed=12, seq_len=180, batch=2)
    tp = 120
    cap = round_up(tp, 32)
    rot = device_rotation(w, inp)
    wp = w.with_len(tp)
    inp_p = dict(inp, k=inp["k"][:, :, :tp].copy(), v=inp["v"][:, :, :tp].copy())
    k, v, oqk, oqv = oracle_caches(wp, inp_p, cap)
    kt = torch.from_numpy(inp["k"][:, :, tp:].copy()).cuda()
    vt = torch.from_numpy(inp["v"][:, :, tp:].copy()).cuda()
    q = torch.from_numpy(inp["q"]).cuda()
    lens_p = np.array([tp, 75], dtype=np.int32)
    lens_t = np.array([60, 0], dtype=np.int32)
    sp, st = 3, 2
    po = torch.empty((sp + st, w.batch, w.n_q_heads, 128), device="cuda")
    pl = torch.empty((sp + st, w.batch, w.n_q_heads), device="cuda")
    tq.decode_attention(rot, k, v, q, seq_lens=torch.from_numpy(lens_p).cuda(), max_len=tp, n_splits=sp,
                        part_o=po[:sp], part_lse=pl[:sp])
    tq.dense_attention(rot, kt, vt, q, seq_lens=torch.from_numpy(lens_t).cuda(), max_len=60, n_splits=st,
                       part_o=po[sp:], part_lse=pl[sp:])
    out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    ref, ref_lse = attention.decode_two_stores(inp["q"].astype(np.float64), dequantized(wp, inp_p, oqk),
                                               dequantized(wp, inp_p, oqv), lens_p, inp["k"][:, :, tp:],
                                               inp["v"][:, :, tp:], lens_t, w.scale)
    err = row_rel_err(out.cpu().numpy(), ref)
    print("packed + tail: max row rel err %.3e" % err.max(), flush=True)
    assert err.max() <= OUT_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("name", list(CASES))
def test_single_token_steps_match_oracle(name):
    # a prefill, then one-token steps through the fused call (its single-token kernel) at
    # host and at device positions, across a tile boundary; neighbours in shared value words
    # must survive every step
    w, inp = setup(name, seed=8, seq_len=70, batch=2)
    t = w.seq_len
    cap = 96
    rot = device_rotation(w, inp)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    k, v = empty_caches(w, cap)
    p1 = 29
    tq.quantize_append_kv(rot, k, v, kx[:, :, :p1].contiguous(), vx[:, :, :p1].contiguous())
    for s in range(p1, t):
        xs, ys = kx[:, :, s:s + 1].contiguous(), vx[:, :, s:s + 1].contiguous()
        if s % 2:
            tq.quantize_append_kv(rot, k, v, xs, ys, pos0=s)
        else:
            pos = torch.full((w.batch,), s, dtype=torch.int32, device="cuda")
            tq.quantize_append_kv(rot, k, v, xs, ys, pos=pos, max_pos=s)
    torch.cuda.synchronize()
    for role, cache in (("k", k), ("v", v)):
        idx, n = download(cache, role)
        check_codes(idx, n, oracle_quantize(w, inp, role), t)
        assert not idx[:, :, t:].any() and not n[:, :, t:].any()


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("n_splits", [1, 3])
@pytest.mark.parametrize("name", list(CASES))
def test_decode_matches_oracle(name, n_splits, schedule):
    w, inp = setup(name, seed=1)
    t = w.seq_len
    cap = round_up(t, 32)
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, cap)
    q = torch.from_numpy(inp["q"]).cuda()
    lens = np.full(w.batch, t)
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref_out, ref_lse = oracle_decode(w, inp, kd, vd, lens)
    if n_splits == 1:
        out, lse = tq.decode_attention(rot, k, v, q, n_splits=1, schedule=schedule, max_len=t)
    else:
        po, pl = tq.decode_attention(rot, k, v, q, n_splits=n_splits, schedule=schedule, max_len=t)
        ref_po, ref_pl = oracle_decode(w, inp, kd, vd, lens, n_splits)
        err_p = row_rel_err(po.cpu().numpy(), ref_po)
        assert err_p.max() <= OUT_RTOL, "partial err %g" % err_p.max()
        np.testing.assert_allclose(pl.cpu().numpy(), ref_pl, rtol=1e-4, atol=1e-4)
        out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    err = row_rel_err(out.cpu().numpy(), ref_out)
    print("max row rel err %.3e (schedule %s, splits %d)" % (err.max(), schedule, n_splits), flush=True)
    assert err.max() <= OUT_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("n_splits", [1, 5, 40])
def test_decode_ragged_lengths_and_empty_rows(n_splits, schedule):
    w, inp = setup("gqa8k", seed=2, seq_len=300, batch=5)
    cap = 320
    lens = np.array([0, 1, 33, 300, 64], dtype=np.int32)
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, cap)
    q = torch.from_numpy(inp["q"]).cuda()
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref_out, ref_lse = attention.decode(inp["q"].astype(np.float64), kd, vd, lens, w.scale)
    seq = torch.from_numpy(lens).cuda()
    if n_splits == 1:
        out, lse = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=300, schedule=schedule)
    else:
        po, pl = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=300, n_splits=n_splits, schedule=schedule)
        out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    assert not out[0].any() and np.all(np.isneginf(lse[0]))
    err = row_rel_err(out[1:], ref_out[1:])
    assert err.max() <= OUT_RTOL
    np.testing.assert_allclose(lse[1:], ref_lse[1:], rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("name", ["gqa8k", "isoquant32k"])
def test_decode_with_distinct_value_codebook(name):
    # 3-bit keys and values normally share one decode table; a value codebook that differs
    # from the key codebook must take the separate-table kernel and still be right
    w, inp = setup(name, seed=10, seq_len=96, batch=2)
    t = w.seq_len
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, t)
    cb = tq.make_codebook(w.bits_v, w.group)
    for i in range(1 << w.bits_v):
        cb.centroid[i] *= 1.01
    v2 = tq.PackedCache(w.batch, w.n_kv_heads, t, w.bits_v, w.group, tq.TQ_VALUES, codes=v.codes, norms=v.norms,
                        codebook=cb)
    oqv2 = dict(oqv)
    oqv2["centroids"] = np.asarray(oqv["centroids"]) * 1.01
    q = torch.from_numpy(inp["q"]).cuda()
    ref, _ = oracle_decode(w, inp, dequantized(w, inp, oqk), dequantized(w, inp, oqv2), np.full(w.batch, t))
    for schedule in ("mfma", "vec"):
        out, _ = tq.decode_attention(rot, k, v2, q, max_len=t, schedule=schedule)
        torch.cuda.synchronize()
        assert row_rel_err(out.cpu().numpy(), ref).max() <= OUT_RTOL
    # 20 sections: 320 workgroups, more than the compute units, so the four-wave kernel runs
    po, pl = tq.decode_attention(rot, k, v2, q, max_len=t, n_splits=20, schedule="mfma")
    out, _ = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy(), ref).max() <= OUT_RTOL


def test_schedules_agree_and_are_deterministic():
    w, inp = setup("gqa8k", seed=3, seq_len=300, batch=1)
    rot = device_rotation(w, inp)
    k, v, _, _ = oracle_caches(w, inp, 320)
    q = torch.from_numpy(inp["q"]).cuda()
    a1, _ = tq.decode_attention(rot, k, v, q, max_len=300, schedule="mfma")
    a2, _ = tq.decode_attention(rot, k, v, q, max_len=300, schedule="mfma")
    b1, _ = tq.decode_attention(rot, k, v, q, max_len=300, schedule="vec")
    torch.cuda.synchronize()
    assert torch.equal(a1, a2)
    assert row_rel_err(a1.cpu().numpy(), b1.cpu().numpy()).max() <= OUT_RTOL


@pytest.mark.parametrize("name,s", [("isoquant32k", 6), ("isoquant32k", 20), ("long128k", 64), ("gqa8k", 1100)])
def test_merge_matches_oracle(name, s):
    # section counts for one, two and four groups of 128 threads, and more sections than the
    # merge keeps weights for in LDS (1024)
    w, inp = setup(name, seed=4, seq_len=32, batch=2)
    rng = np.random.default_rng(5)
    bsz, hq = w.batch, w.n_q_heads
    po = rng.standard_normal((s, bsz, hq, 128)).astype(np.float32)
    pl = (rng.standard_normal((s, bsz, hq)) * 5).astype(np.float32)
    pl[2] = -np.inf                       # an empty split everywhere
    pl[:, 1, 3] = -np.inf                 # a row with no tokens at all
    rot = device_rotation(w, inp)
    out, lse = tq.merge_splits(rot, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    m_out, m_lse = attention.merge(po, pl)
    ref = np.empty_like(m_out)
    for h in range(hq):
        kv = h // w.group_size
        ref[:, h] = rotation.unrotate(m_out[:, h], inp["signs"][kv], w.group,
                                      None if inp["so4"] is None else inp["so4"][kv])
    err = row_rel_err(out.cpu().numpy(), ref)
    assert err.max() <= 1e-5
    np.testing.assert_allclose(lse.cpu().numpy(), m_lse, rtol=1e-6, atol=1e-6)
    assert not out.cpu().numpy()[1, 3].any()


@pytest.mark.parametrize("name", ["gqa8k", "isoquant32k"])
def test_end_to_end_append_then_decode(name):
    w, inp = setup(name, seed=6)
    t = w.seq_len
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, round_up(t, 32))
    tq.quantize_append(rot, k, torch.from_numpy(inp["k"]).cuda())
    tq.quantize_append(rot, v, torch.from_numpy(inp["v"]).cuda())
    out, _ = tq.decode_attention(rot, k, v, torch.from_numpy(inp["q"]).cuda(), max_len=t)
    torch.cuda.synchronize()
    oqk, oqv = oracle_quantize(w, inp, "k"), oracle_quantize(w, inp, "v")
    ref, _ = oracle_decode(w, inp, dequantized(w, inp, oqk), dequantized(w, inp, oqv), np.full(w.batch, t))
    assert row_rel_err(out.cpu().numpy(), ref).max() <= OUT_RTOL


def scaled_values(inp, vscale, seed):
    """The workload's values (fp32) times a scale: a constant, or per token 10^u with u uniform
    in [-4, 4] ("mixed": value group norms spanning eight decades inside one row)."""
    v = inp["v"].astype(np.float32)
    if vscale == "mixed":
        rng = np.random.default_rng(seed)
        return (v * 10.0 ** rng.uniform(-4, 4, size=v.shape[:3] + (1,))).astype(np.float32)
    return (v * np.float32(vscale)).astype(np.float32)


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("vscale", [1e-4, 1e4, "mixed"])
@pytest.mark.parametrize("name", ["gqa8k", "batched", "long128k", "isoquant32k"])
def test_decode_value_scales(name, vscale, schedule):
    # The norm is stored apart from the unit vector ("TurboQuant ...", 2.1), so a value group
    # norm can be any fp32 number; the matrix-core schedule rounds the value weights p * norm
    # to fp16 and must keep them in range at any scale.  Ragged rows and key-axis sections
    # with empty ones exercise the masked slots.
    w, inp = setup(name, seed=13, seq_len=150, batch=2)
    inp = dict(inp, v=scaled_values(inp, vscale, 13))
    if vscale == "mixed":
        # With value norms spread over eight decades a row's output can be carried by a token
        # whose softmax weight is 1e-6; the row error is then that token's absolute score
        # error, which for the workloads' outlier keys reaches 1e-3 on the matrix-core path
        # (fp16 codebook levels at their fp16-exact scale).  Keys at a quarter of their size
        # keep scores within a few units, so this case measures the value weights' range.
        inp["k"] = (inp["k"].astype(np.float32) * np.float32(0.25)).astype(np.float32)
    t = w.seq_len
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, round_up(t, 32))
    q = torch.from_numpy(inp["q"]).cuda()
    lens = np.array([t, 37], dtype=np.int32)
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref_out, ref_lse = oracle_decode(w, inp, kd, vd, lens)
    seq = torch.from_numpy(lens).cuda()
    for n_splits in (1, 3, 8):
        if n_splits == 1:
            out, lse = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, schedule=schedule)
        else:
            po, pl = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, n_splits=n_splits, schedule=schedule)
            out, lse = tq.merge_splits(rot, po, pl)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.isfinite(o).all()
        err = row_rel_err(o, ref_out)
        print("value scale %s, splits %d: max row rel err %.3e" % (vscale, n_splits, err.max()), flush=True)
        assert err.max() <= OUT_RTOL
        np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


def zero_code(bits):
    # a zero group normalises to y = 0; its code counts the boundaries strictly below 0
    # (the middle boundary is 0 itself), i.e. 2^(bits-1) - 1
    return (1 << (bits - 1)) - 1


@pytest.mark.parametrize("name", list(CASES))
def test_zero_groups_append_and_decode(name):
    # Zero groups store norm 0 and the code of y = 0, and decode to zero: whole zero tokens,
    # a zero 32-coordinate group inside otherwise nonzero tokens, and a zero last token, in
    # keys and values, appended in one call and one token at a time; then both schedules
    # against the oracle on those caches.
    w, inp = setup(name, seed=14, seq_len=100, batch=2)
    kx, vx = inp["k"].astype(np.float32), inp["v"].astype(np.float32)
    kx[0, :, 5] = 0.0
    vx[0, :, 5] = 0.0
    kx[1, :, 40:45, 32:64] = 0.0
    vx[1, :, 60:63, 96:128] = 0.0
    vx[0, :, 10:12] = 0.0
    kx[:, :, 99] = 0.0
    vx[:, :, 99] = 0.0
    inp = dict(inp, k=kx, v=vx)
    t = w.seq_len
    cap = round_up(t, 32)
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, cap)
    kt, vt = torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda()
    tq.quantize_append_kv(rot, k, v, kt[:, :, :t - 1].contiguous(), vt[:, :, :t - 1].contiguous())
    tq.quantize_append_kv(rot, k, v, kt[:, :, t - 1:].contiguous(), vt[:, :, t - 1:].contiguous(), pos0=t - 1)
    torch.cuda.synchronize()
    for role, cache, x in (("k", k, kx), ("v", v, vx)):
        oq = oracle_quantize(w, inp, role)
        idx, n = download(cache, role)
        zero = (np.abs(x.reshape(x.shape[:3] + (128 // w.group, w.group))).max(-1) == 0)
        assert zero.any()
        assert np.all(n[:, :, :t][zero] == 0.0) and np.all(oq["norms"][zero] == 0.0)
        zc = np.repeat(zero, w.group, axis=-1)
        assert np.all(idx[:, :, :t][zc] == zero_code(cache.bits)) and np.all(oq["idx"][zc] == zero_code(cache.bits))
        check_codes(idx, n, oq, t)
    q = torch.from_numpy(inp["q"]).cuda()
    oqk, oqv = oracle_quantize(w, inp, "k"), oracle_quantize(w, inp, "v")
    ref, ref_lse = oracle_decode(w, inp, dequantized(w, inp, oqk), dequantized(w, inp, oqv), np.full(w.batch, t))
    for schedule in ("mfma", "vec"):
        for n_splits in (1, 4):
            if n_splits == 1:
                out, lse = tq.decode_attention(rot, k, v, q, max_len=t, schedule=schedule)
            else:
                po, pl = tq.decode_attention(rot, k, v, q, max_len=t, n_splits=n_splits, schedule=schedule)
                out, lse = tq.merge_splits(rot, po, pl)
            torch.cuda.synchronize()
            err = row_rel_err(out.cpu().numpy(), ref)
            print("zero groups: schedule %s splits %d: max row rel err %.3e" % (schedule, n_splits, err.max()),
                  flush=True)
            assert err.max() <= OUT_RTOL
            np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("name,n_q_heads", [("long128k", 16), ("batched", 64), ("gqa8k", 48), ("gqa8k", 128)])
def test_decode_more_than_four_heads_per_kv_head(name, n_q_heads, schedule):
    # more query heads per KV head than one workgroup serves: 32-coordinate groups take 4 heads
    # per workgroup, so G = 6, 8 and 16 run in 2, 2 and 4 head slices (the last one partial for
    # G = 6), for the shared 3-bit table and for 4-bit keys with 3-bit values; ragged rows and
    # sections
    from dataclasses import replace
    w = replace(workloads.WORKLOADS[name], n_q_heads=n_q_heads).with_len(130, batch=2)
    inp = workloads.generate(w, 15)
    print("case", name, "G", w.group_size, flush=True)
    t = w.seq_len
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, round_up(t, 32))
    q = torch.from_numpy(inp["q"]).cuda()
    lens = np.array([t, 45], dtype=np.int32)
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref_out, ref_lse = oracle_decode(w, inp, kd, vd, lens)
    seq = torch.from_numpy(lens).cuda()
    for n_splits in (1, 3):
        if n_splits == 1:
            out, lse = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, schedule=schedule)
        else:
            po, pl = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, n_splits=n_splits, schedule=schedule)
            ref_po, ref_pl = oracle_decode(w, inp, kd, vd, lens, n_splits)
            assert row_rel_err(po.cpu().numpy(), ref_po).max() <= OUT_RTOL
            np.testing.assert_allclose(pl.cpu().numpy(), ref_pl, rtol=1e-4, atol=1e-4)
            out, lse = tq.merge_splits(rot, po, pl)
        torch.cuda.synchronize()
        err = row_rel_err(out.cpu().numpy(), ref_out)
        print("splits %d: max row rel err %.3e" % (n_splits, err.max()), flush=True)
        assert err.max() <= OUT_RTOL
        np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("bits_k,bits_v,group_size,so4", [(4, 4, 1, True), (4, 3, 3, True), (3, 4, 8, False),
                                                          (3, 3, 12, True), (4, 4, 16, False)])
def test_whole_head_groups_bits_and_head_counts(bits_k, bits_v, group_size, so4, schedule):
    # 128-coordinate groups with every pair of code widths (two-code tables for 4-bit codes,
    # the shared four-code table for 3/3), with and without SO(4) blocks, and query groups of
    # 1, 3, 8, 12 and 16 heads per KV head (one head slice of up to 8: partial, full, a full
    # and a partial one, two); 10 sections of 4 rows x 8 KV heads give more workgroups than
    # compute units (the four-wave instance), 1 and 3 sections the eight-wave one
    from dataclasses import replace
    w = replace(workloads.WORKLOADS["isoquant32k"], bits_k=bits_k, bits_v=bits_v, so4=so4,
                n_q_heads=8 * group_size).with_len(150, batch=4)
    inp = workloads.generate(w, 21)
    print("case bits %d/%d G %d so4 %s" % (bits_k, bits_v, group_size, so4), flush=True)
    t = w.seq_len
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, round_up(t, 32))
    q = torch.from_numpy(inp["q"]).cuda()
    lens = np.array([t, 45, 0, 97], dtype=np.int32)
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref_out, ref_lse = oracle_decode(w, inp, kd, vd, lens)
    seq = torch.from_numpy(lens).cuda()
    # The matrix-core schedule holds the codebook levels as fp16 numbers (relative error at
    # most 3e-5 for 3-bit and 1e-4 for 4-bit levels, checked on the CPU), so a score moves by
    # at most that times scale * |q| * |k_hat| (Cauchy-Schwarz), and an lse by at most the
    # largest such bound of its row: these inputs reach scores near 30, where that passes 1e-4.
    eps = 3e-5 if bits_k == 3 else 1e-4
    qn = np.linalg.norm(inp["q"].astype(np.float64), axis=-1)                      # [B, Hq]
    kmax = np.linalg.norm(kd, axis=-1).max(axis=-1).repeat(group_size, axis=1)      # [B, Hq]
    lse_atol = 1e-4 + (eps * w.scale * qn * kmax if schedule == "mfma" else 0.0 * qn)
    for n_splits in (1, 3, 10):
        if n_splits == 1:
            out, lse = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, schedule=schedule)
        else:
            po, pl = tq.decode_attention(rot, k, v, q, seq_lens=seq, max_len=t, n_splits=n_splits, schedule=schedule)
            ref_po, ref_pl = oracle_decode(w, inp, kd, vd, lens, n_splits)
            assert row_rel_err(po.cpu().numpy(), ref_po).max() <= OUT_RTOL
            gp, live_s = pl.cpu().numpy(), np.isfinite(ref_pl)
            assert np.array_equal(np.isfinite(gp), live_s)  # empty sections: -inf
            assert np.all(np.abs(gp[live_s] - ref_pl[live_s]) <= np.broadcast_to(lse_atol, ref_pl.shape)[live_s])
            out, lse = tq.merge_splits(rot, po, pl)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        assert not o[2].any() and np.all(l[2] == -np.inf)  # the empty row
        live = [0, 1, 3]
        err = row_rel_err(o[live], ref_out[live])
        dl = np.abs(l[live] - ref_lse[live])
        print("splits %d: max row rel err %.3e, lse err %.2e (bound %.2e)" % (n_splits, err.max(), dl.max(),
                                                                          lse_atol[live].min()), flush=True)
        assert err.max() <= OUT_RTOL
        assert np.all(dl <= lse_atol[live])

@pytest.mark.parametrize("schedule", ["mfma", "vec"])
@pytest.mark.parametrize("t", [32, 511, 512, 513])
def test_decode_both_schedules_around_the_pages_threshold(t, schedule):
    # the pages switch the value accumulation from word- to dimension-parallel at T = 512; here
    # the matrix-core schedule is faster at every T measured, and both schedules must hold the
    # bar on either side of that length
    w, inp = setup("gqa8k", seed=16, seq_len=t, batch=1)
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, round_up(t, 32))
    ref, ref_lse = oracle_decode(w, inp, dequantized(w, inp, oqk), dequantized(w, inp, oqv), np.full(1, t))
    out, lse = tq.decode_attention(rot, k, v, torch.from_numpy(inp["q"]).cuda(), max_len=t, schedule=schedule)
    torch.cuda.synchronize()
    assert row_rel_err(out.cpu().numpy(), ref).max() <= OUT_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-4, atol=1e-4)


def test_binding_refuses_mismatched_buffers():
    # buffers the kernels would address past their end, or in another type, are refused by the
    # binding before any launch (host-side checks only; nothing runs on the device)
    w, inp = setup("gqa8k", seq_len=64, batch=2)
    rot = device_rotation(w, inp)
    k, v = empty_caches(w, 64)
    q = torch.from_numpy(inp["q"]).cuda()
    x = torch.from_numpy(inp["k"]).cuda()
    bad = [
        lambda: tq.decode_attention(rot, k, v, q[:1]),                                    # fewer rows than the cache
        lambda: tq.decode_attention(rot, k, v, q[..., :64].contiguous()),                 # not 128 wide
        lambda: tq.decode_attention(rot, k, v, q, seq_lens=torch.zeros(1, dtype=torch.int32, device="cuda")),
        lambda: tq.decode_attention(rot, k, v, q, seq_lens=torch.zeros(2, dtype=torch.int64, device="cuda")),
        lambda: tq.decode_attention(rot, k, v, q, out=torch.empty(2, w.n_q_heads, 64, device="cuda")),
        lambda: tq.decode_attention(rot, k, v, q, n_splits=3, part_o=torch.empty(2, 2, w.n_q_heads, 128, device="cuda")),
        lambda: tq.quantize_append(rot, k, x[:1].contiguous()),                           # fewer rows
        lambda: tq.quantize_append(rot, k, x, pos=torch.zeros(3, dtype=torch.int32, device="cuda")),
        lambda: tq.quantize_append_kv(rot, k, v, x[:, :1].contiguous(), x[:, :1].contiguous()),  # fewer KV heads
        lambda: tq.append_decode_attention(rot, k, v, x[:, :, :1].contiguous(), x[:, :, :1].contiguous(), q[:1],
                                           pos0=10),
        lambda: tq.merge_splits(rot, torch.empty(3, 2, w.n_q_heads, 128, device="cuda"),
                                torch.empty(3, 2, w.n_q_heads + 1, device="cuda")),
        lambda: tq.decode_attention(rot, k, v, q.cpu()),                                  # host memory
    ]
    for i, call in enumerate(bad):
        with pytest.raises(ValueError):
            call()
        torch.cuda.synchronize()
    # the well-formed call still runs
    tq.quantize_append_kv(rot, k, v, x, torch.from_numpy(inp["v"]).cuda())
    out, lse = tq.decode_attention(rot, k, v, q, max_len=64)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("bits_k,bits_v,group,so4", [(4, 3, 32, False), (3, 3, 128, True)])
def test_vector_schedule_on_extreme_scores(bits_k, bits_v, group, so4):
    # Two 10x channels shared by queries and keys put scores near 86; the matrix-core schedule's
    # fp16 key levels then move output rows by 2-3e-3 (the library header states this limit),
    # while the vector schedule, fp32 throughout, holds the bar.  The matrix-core rows are
    # checked against the level-error bound instead.
    from dataclasses import replace
    w = replace(workloads.WORKLOADS["isoquant32k"], bits_k=bits_k, bits_v=bits_v, group=group, so4=so4,
                outliers="fixed2x10", n_q_heads=32).with_len(512, batch=2)
    inp = workloads.generate(w, 5)
    rot = device_rotation(w, inp)
    k, v, oqk, oqv = oracle_caches(w, inp, 512)
    q = torch.from_numpy(inp["q"]).cuda()
    kd, vd = dequantized(w, inp, oqk), dequantized(w, inp, oqv)
    ref, ref_lse = oracle_decode(w, inp, kd, vd, np.full(2, 512))
    out, lse = tq.decode_attention(rot, k, v, q, max_len=512, schedule="vec")
    torch.cuda.synchronize()
    err = row_rel_err(out.cpu().numpy(), ref)
    print("vector schedule: max row rel err %.2e, max |lse| %.1f" % (err.max(), np.abs(ref_lse).max()), flush=True)
    assert np.abs(ref_lse).max() > 60  # the case is the one the header describes
    assert err.max() <= OUT_RTOL
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-4)
    out, lse = tq.decode_attention(rot, k, v, q, max_len=512, schedule="mfma")
    torch.cuda.synchronize()
    eps = 3e-5 if bits_k == 3 else 1e-4
    bound = eps * w.scale * np.linalg.norm(inp["q"].astype(np.float64), axis=-1) * \
        np.linalg.norm(kd, axis=-1).max(axis=-1).repeat(w.group_size, axis=1)
    dl = np.abs(lse.cpu().numpy() - ref_lse)
    print("matrix cores: max row rel err %.2e, lse err %.2e (bound %.2e)" % (
        row_rel_err(out.cpu().numpy(), ref).max(), dl.max(), bound.min()), flush=True)
    assert np.all(dl <= 1e-4 + bound)

"""Seeded random configurations of the unquantised region, Block-GTQ keys, two-stage keys and
lossless BF16 pages through the C ABI against the oracle: head counts and groupings, ragged
rows (an empty one now and then), section counts, dtypes and, for Block-GTQ, the width range
and bit budget of the allocation.  Block-GTQ and two-stage keys are encoded by the library in
two calls cut at a random slot and compared with the oracle's records; attention runs on the
oracle's records.  BF16 pages are compressed in two calls cut at a random page, must equal the
oracle's store and metadata byte for byte, and attention reads the library's pages."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import oracle_decode, row_rel_err
from oracle import blockgtq as bg, qjl, zipcodec as zc

pytestmark = pytest.mark.gpu

DENSE_RTOL = 1e-4  # fp32 scores and sums over unquantised inputs
FLIPS = {"flips": 0, "coords": 0, "cases": 0}  # code flips near a boundary, pooled over cases
N_GTQ, N_QJL, N_ZIP = 12, 8, 12


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


def ragged(rng, batch, t):
    """Row lengths in [0, t]: one row of t tokens, and now and then an empty one."""
    lens = rng.integers(0, t + 1, size=batch).astype(np.int32)
    full = int(rng.integers(0, batch))
    lens[full] = t
    if batch > 1 and rng.integers(0, 3) == 0:
        lens[(full + 1 + int(rng.integers(0, batch - 1))) % batch] = 0
    return lens


@pytest.mark.parametrize("seed", range(16))
def test_random_dense(seed):
    rng = np.random.default_rng(8000 + seed)
    group = int(rng.choice([32, 128]))
    hkv, g = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5, 8, 12, 16, 24]))
    t = int(rng.integers(1, 301))
    w = replace(workloads.WORKLOADS["isoquant32k"], batch=int(rng.integers(1, 4)), n_kv_heads=hkv,
                n_q_heads=g * hkv, seq_len=t, group=group, so4=bool(rng.integers(0, 2)))
    kv_dtype, q_dtype = rng.choice([np.float16, np.float32]), rng.choice([np.float16, np.float32])
    n_splits = int(rng.choice([1, 2, 3, 7, 16]))
    lens = ragged(rng, w.batch, t)
    print("dense case %d: B=%d Hq=%d Hkv=%d T=%d g=%d so4=%s kv %s q %s lens %s S=%d" % (
        seed, w.batch, w.n_q_heads, hkv, t, group, w.so4, np.dtype(kv_dtype).name, np.dtype(q_dtype).name,
        list(lens), n_splits), flush=True)
    inp = workloads.generate(w, seed)
    kx, vx = inp["k"].astype(kv_dtype), inp["v"].astype(kv_dtype)
    inp = dict(inp, q=inp["q"].astype(q_dtype))
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).cuda()
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), group, so4)
    po, pl = tq.dense_attention(rot, torch.from_numpy(kx).cuda(), torch.from_numpy(vx).cuda(),
                                torch.from_numpy(inp["q"]).cuda(), seq_lens=torch.from_numpy(lens).cuda(), max_len=t,
                                n_splits=n_splits)
    out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_decode(w, inp, kx.astype(np.float64), vx.astype(np.float64), lens)
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    live = lens > 0
    assert not o[~live].any() and np.all(l[~live] == -np.inf)
    err = row_rel_err(o[live], ref[live])
    print("   max row rel err %.2e" % err.max(initial=0), flush=True)
    assert err.max(initial=0) <= DENSE_RTOL
    np.testing.assert_allclose(l[live], ref_lse[live], rtol=1e-5, atol=1e-5)


def gtq_draw(seed):
    rng = np.random.default_rng(9000 + seed)
    b_min = int(rng.integers(1, 6))
    b_max = min(8, b_min + int(rng.integers(0, 4)))
    budget = int(rng.integers(64 * b_min, 64 * b_max + 1))
    hkv, g = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 4, 8, 16]))
    batch = int(rng.integers(1, 4))
    cap = int(rng.integers(1, 10)) * 32
    t = int(rng.integers(1, cap + 1))
    return rng, (b_min, b_max, budget), hkv, g, batch, cap, t


def record_check(got, ref, ys, enc, n_tokens):
    """Every code that differs from the oracle's lies within 1e-6 of its group's boundary."""
    bad = got[:, :, :n_tokens] != ref[:, :, :n_tokens]
    for b, h, tk, j in zip(*np.nonzero(bad)):
        ends = np.cumsum([len(e[1]) for e in enc[h]])
        m = enc[h][int(np.searchsorted(ends, j, side="right"))][4]
        assert np.min(np.abs(m - ys[b, h, tk, j])) < 1e-6, (b, h, tk, j)
    FLIPS["flips"] += int(bad.sum())
    FLIPS["coords"] += bad.size


@pytest.mark.parametrize("seed", range(N_GTQ))
def test_random_gtq(seed):
    from test_gpu_gtq import check, oracle_attention, oracle_keys, pack_records, unpack_records
    rng, widths, hkv, g, batch, cap, t = gtq_draw(seed)
    lens = ragged(rng, batch, t)
    n_splits = int(rng.choice([1, 2, 3, 7, 16]))
    q_dtype = rng.choice([np.float16, np.float32])
    w = replace(workloads.WORKLOADS["gtq32k"], batch=batch, n_q_heads=g * hkv, n_kv_heads=hkv, seq_len=cap)
    print("gtq case %d: B=%d Hq=%d Hkv=%d cap=%d widths %s lens %s S=%d q %s" % (
        seed, batch, g * hkv, hkv, cap, widths, list(lens), n_splits, np.dtype(q_dtype).name), flush=True)
    inp = workloads.generate(w, seed)
    s = bg.block_energies(inp["q_cal"], inp["k_cal"]).astype(np.float32)
    bits = np.stack([bg.allocate(s[h].astype(np.float64), widths[2], widths[0], widths[1]) for h in range(hkv)])
    if any(len(set(bits[h].tolist())) > 4 for h in range(hkv)):
        pytest.skip("an allocation with more than four widths in a head (refused by the library)")
    enc = [bg.head_encoders(bits[h], inp["gauss"][h].astype(np.float64)) for h in range(hkv)]
    keys = tq.GtqKeys(bits, inp["gauss"])
    cb = keys.code_bytes
    # the library's encoding in two calls, against the oracle's records
    codes = torch.zeros((batch, hkv, cap, cb), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((batch, hkv, cap, 4), dtype=torch.float32, device="cuda")
    x = torch.from_numpy(inp["k"]).cuda()
    cut = int(rng.integers(0, cap + 1))
    if cut > 0:
        tq.gtq_quantize_keys(keys, x[:, :, :cut].contiguous(), codes, norms, pos0=0)
    if cut < cap:
        tq.gtq_quantize_keys(keys, x[:, :, cut:].contiguous(), codes, norms, pos0=cut)
    torch.cuda.synchronize()
    oc, on, oy = oracle_keys(w, inp, enc)
    record_check(unpack_records(codes.cpu().numpy(), enc), oc, oy, enc, cap)
    assert np.allclose(norms.cpu().numpy(), on, rtol=1e-6, atol=1e-30)
    # attention on the oracle's records
    codes = torch.from_numpy(pack_records(oc, enc, cb)).cuda()
    v = torch.from_numpy(inp["v"].astype(np.float16)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16).astype(q_dtype)).cuda()
    inp = dict(inp, q=inp["q"].astype(np.float16).astype(np.float64))
    res = tq.gtq_attention(keys, codes, torch.from_numpy(on).cuda(), v, q, seq_lens=torch.from_numpy(lens).cuda(),
                           max_len=t, scale=w.scale, n_splits=n_splits)
    if n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    (ro, rl), _ = oracle_attention(w, inp, enc, oc, on, lens)
    check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, lens)
    FLIPS["cases"] += 1


@pytest.mark.parametrize("seed", range(N_QJL))
def test_random_qjl(seed):
    from test_gpu_qjl import check, oracle_records
    rng = np.random.default_rng(9500 + seed)
    bits_k = int(rng.integers(2, 5))
    hkv, g = int(rng.integers(1, 4)), int(rng.choice([1, 2, 4, 8, 16]))
    batch = int(rng.integers(1, 4))
    cap = int(rng.integers(1, 10)) * 32
    t = int(rng.integers(1, cap + 1))
    lens = ragged(rng, batch, t)
    n_splits = int(rng.choice([1, 2, 3, 7]))
    w = replace(workloads.WORKLOADS["qjl32k"], batch=batch, n_q_heads=g * hkv, n_kv_heads=hkv, seq_len=cap,
                bits_k=bits_k)
    print("qjl case %d: B=%d Hq=%d Hkv=%d cap=%d bits %d lens %s S=%d" % (
        seed, batch, g * hkv, hkv, cap, bits_k, list(lens), n_splits), flush=True)
    inp = workloads.generate(w, seed)
    bits = bits_k - 1
    enc = [qjl.mse_encoders(bits, inp["gauss"][h].astype(np.float64)) for h in range(hkv)]
    keys = tq.QjlKeys(bits, inp["gauss"], inp["proj"])
    cb = keys.code_bytes
    oc, on, osg, orn, oxh = oracle_records(w, inp, enc)
    # the library's first-stage codes and norms from two calls, against the oracle's
    codes = torch.zeros((batch, hkv, cap, cb), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((batch, hkv, cap, 4), dtype=torch.float32, device="cuda")
    signs = torch.zeros((batch, hkv, cap, 16), dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(inp["k"]).cuda()
    cut = int(rng.integers(0, cap + 1))
    if cut > 0:
        tq.qjl_quantize_keys(keys, x[:, :, :cut].contiguous(), codes, norms, signs, pos0=0)
    if cut < cap:
        tq.qjl_quantize_keys(keys, x[:, :, cut:].contiguous(), codes, norms, signs, pos0=cut)
    torch.cuda.synchronize()
    got = qjl.unpack_codes(codes.cpu().numpy().reshape(-1, cb), bits).reshape(oc.shape)
    ys = np.zeros(oc.shape)
    for b in range(batch):
        for h in range(hkv):
            ys[b, h] = bg.quantize_keys(inp["k"][b, h].astype(np.float64), enc[h])[2]
    record_check(got, oc, ys, enc, cap)
    assert np.allclose(norms.cpu().numpy()[..., 0], on[..., 0], rtol=1e-6, atol=0)
    # attention on the oracle's records
    packed = qjl.pack_codes(oc.reshape(-1, 128), bits).reshape(oc.shape[:3] + (cb,))
    v = torch.from_numpy(inp["v"].astype(np.float16)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16)).cuda()
    res = tq.qjl_attention(keys, torch.from_numpy(packed).cuda(), torch.from_numpy(on).cuda(),
                           torch.from_numpy(osg).cuda(), v, q, seq_lens=torch.from_numpy(lens).cuda(), max_len=t,
                           scale=w.scale, n_splits=n_splits)
    if n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    ro = np.zeros((batch, w.n_q_heads, 128))
    rl = np.full((batch, w.n_q_heads), -np.inf)
    vf = inp["v"].astype(np.float16).astype(np.float64)
    for b, tt in enumerate(lens):
        if tt == 0:
            continue
        for h in range(w.n_q_heads):
            kv = h // w.group_size
            S = inp["proj"][kv].astype(np.float64)
            qv = inp["q"][b, h].astype(np.float16).astype(np.float64)
            s = w.scale * qjl.scores(qv, oxh[b, kv, :tt], osg[b, kv, :tt], orn[b, kv, :tt], S)
            m = s.max()
            p = np.exp(s - m)
            ro[b, h] = (p / p.sum()) @ vf[b, kv, :tt]
            rl[b, h] = m + np.log(p.sum())
    check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, lens)
    FLIPS["cases"] += 1


def exponent_windows(rng, x, pages, role):
    """Set the exponents of a few random chunks of x (BF16 bits [B, H, T, 128]) to a window
    of width 14 to 17 from an even or odd base, touching both ends: chunks at and just past
    the largest coded span."""
    for _ in range(int(rng.integers(0, 9))):
        b, h, p = (int(rng.integers(0, n)) for n in x.shape[:2] + (pages,))
        vals = zc.page_values(x[b, h, zc.PAGE * p:zc.PAGE * (p + 1)], role).reshape(zc.CHUNKS, zc.CHUNK)
        c, lo, span = int(rng.integers(0, zc.CHUNKS)), int(rng.integers(100, 113)), int(rng.integers(14, 18))
        e = lo + rng.integers(0, span + 1, size=zc.CHUNK)
        e[rng.permutation(zc.CHUNK)[:2]] = (lo, lo + span)
        vals[c] = (vals[c] & 0x807F) | (e.astype(np.uint16) << 7)
        x[b, h, zc.PAGE * p:zc.PAGE * (p + 1)] = zc.page_from_values(vals.reshape(-1), role)


@pytest.mark.parametrize("seed", range(N_ZIP))
def test_random_zip(seed):
    from test_gpu_zip import ROLE, check_rows, dev_bf16, oracle_stores
    rng = np.random.default_rng(9700 + seed)
    hkv, g = int(rng.integers(1, 4)), int(rng.choice([1, 2, 3, 5, 8, 16, 24]))
    batch, pages = int(rng.integers(1, 4)), int(rng.integers(1, 21))
    open_tail = bool(rng.integers(0, 2))
    # an open page past the store's last page when the tail is a 16-row buffer
    t = int(rng.integers(1, zc.PAGE * pages + (zc.PAGE if open_tail else 1)))
    lens = ragged(rng, batch, t)
    n_splits = int(rng.choice([1, 2, 3, 7, 16]))
    q_dtype = [torch.bfloat16, torch.float32, torch.float16][int(rng.integers(0, 3))]
    scale = float(rng.uniform(0.04, 0.12))
    w = replace(workloads.WORKLOADS["zipfusion8k"], batch=batch, n_q_heads=g * hkv, n_kv_heads=hkv,
                seq_len=zc.PAGE * (pages + 1))
    print("zip case %d: B=%d Hq=%d Hkv=%d pages %d lens %s S=%d q %s scale %.3f %s tail" % (
        seed, batch, g * hkv, hkv, pages, lens.tolist(), n_splits, q_dtype, scale,
        "open-page" if open_tail else "whole-cache"), flush=True)
    inp = workloads.generate(w, seed)
    for role in ("k", "v"):
        exponent_windows(rng, inp[role], pages, role)
    # the library's stores from two calls cut at a random page, against the oracle's
    cut = int(rng.integers(0, pages + 1))
    dev = {}
    for role in ("k", "v"):
        s, m = tq.zip_store(batch, hkv, pages)
        x = dev_bf16(inp[role])
        if cut > 0:
            tq.zip_compress(x, s, m, ROLE[role], n_pages=cut)
        if cut < pages:
            tq.zip_compress(x, s, m, ROLE[role], n_pages=pages - cut, src_page0=cut, dst_page0=cut)
        os_, om = oracle_stores(inp[role], pages, role)
        assert np.array_equal(m.cpu().numpy(), om), role
        assert np.array_equal(s.cpu().numpy(), os_), role
        dev[role] = (s, m)
    # tails: the whole BF16 cache, or 16-row buffers holding each row's open page
    if open_tail:
        tails = {r: np.zeros((batch, hkv, zc.PAGE, 128), np.uint16) for r in ("k", "v")}
        for b, n in enumerate(lens):
            for i in range(zc.PAGE * (int(n) // zc.PAGE), int(n)):
                for r in ("k", "v"):
                    tails[r][b, :, i % zc.PAGE] = inp[r][b, :, i]
    else:
        tails = {r: inp[r][:, :, :zc.PAGE * pages] for r in ("k", "v")}
    qb = dev_bf16(inp["q"])
    q = qb if q_dtype == torch.bfloat16 else qb.float().to(q_dtype)
    res = tq.zip_attention(dev["k"][0], dev["k"][1], dev["v"][0], dev["v"][1], dev_bf16(tails["k"]),
                           dev_bf16(tails["v"]), q, seq_lens=torch.from_numpy(lens).cuda(), max_len=t, scale=scale,
                           n_splits=n_splits)
    if n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    ks, km = oracle_stores(inp["k"], pages, "k")
    vs, vm = oracle_stores(inp["v"], pages, "v")
    ref_o, ref_l = zc.decode_from_pages(inp["q"], ks, km, vs, vm, tails["k"], tails["v"], lens, scale)
    check_rows(res[0].cpu().numpy(), res[1].cpu().numpy(), ref_o, ref_l, lens, g)


def test_random_codecs_flip_rate():
    # the code bar's rate (near-boundary flips at most 1e-5 of all coordinates) pooled over the
    # Block-GTQ and two-stage cases of the session
    if FLIPS["cases"] < N_GTQ + N_QJL - 2:
        pytest.skip("the rate is pooled over the random Block-GTQ and two-stage cases of one run")
    print("near-boundary flips: %d of %d coordinates" % (FLIPS["flips"], FLIPS["coords"]), flush=True)
    assert FLIPS["flips"] <= 1e-5 * FLIPS["coords"]

"""GPU parity of the lossless BF16 exponent codec and of attention read from its pages,
through the C ABI, against the oracle (oracle/zipcodec.py).

The compressed store and metadata must equal the oracle's byte for byte (integer work).
Attention outputs are fp32 sums of exact BF16 values: within 1e-4 relative per row of the
fp64 oracle (the unquantised-store bar), lse within 1e-4 absolute.  Rows are ragged: a row
with several pages and an open page, one of whole pages only, one shorter than a page and
an empty one.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import row_rel_err
from oracle import attention, zipcodec as zc

pytestmark = pytest.mark.gpu

RTOL = 1e-4
LSE_ATOL = 1e-4
LENS = [309, 160, 7, 0]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


def case(hq=32, hkv=8, lens=LENS, cap=320, seed=0):
    w = replace(workloads.WORKLOADS["zipfusion8k"], batch=len(lens), n_q_heads=hq, n_kv_heads=hkv, seq_len=cap)
    inp = workloads.generate(w, seed)
    print("zip case", (len(lens), hq, hkv, cap), "lens", lens, "seed", seed, flush=True)
    return w, inp


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


ROLE = {"k": tq.TQ_KEYS, "v": tq.TQ_VALUES}


def oracle_stores(x, pages, role):
    bsz, hkv = x.shape[:2]
    store = np.zeros((bsz, hkv, pages, zc.SLOT), np.uint8)
    meta = np.zeros((bsz, hkv, pages, 8), np.uint8)
    for b in range(bsz):
        for h in range(hkv):
            store[b, h], meta[b, h] = zc.compress_stream(x[b, h], pages, role)
    return store, meta


def device_stores(x, pages, role):
    s, m = tq.zip_store(x.shape[0], x.shape[1], pages)
    tq.zip_compress(dev_bf16(x), s, m, ROLE[role], n_pages=pages)
    return s, m


@pytest.mark.parametrize("seed", [0, 1])
def test_compress_matches_oracle_bytes(seed):
    w, inp = case(seed=seed)
    pages = w.seq_len // zc.PAGE
    k = inp["k"].copy()
    # chunk 0 of page 2 of stream (0, 0): exponents span exactly 16 (b = 120, max 135): coded;
    # chunk 1 of the same page: span 17 (b = 120, max 136): kept
    k[0, 0, 32:36] = (k[0, 0, 32:36] & 0x807F) | (125 << 7)
    k[0, 0, 32, 0] = (k[0, 0, 32, 0] & 0x807F) | (121 << 7)
    k[0, 0, 33, 1] = (k[0, 0, 33, 1] & 0x807F) | (135 << 7)
    k[0, 0, 36:40] = (k[0, 0, 36:40] & 0x807F) | (125 << 7)
    k[0, 0, 36, 0] = (k[0, 0, 36, 0] & 0x807F) | (120 << 7)
    k[0, 0, 37, 1] = (k[0, 0, 37, 1] & 0x807F) | (136 << 7)
    for x, role in ((k, "k"), (inp["v"], "v")):
        os_, om = oracle_stores(x, pages, role)
        ds, dm = device_stores(x, pages, role)
        assert np.array_equal(dm.cpu().numpy(), om)
        assert np.array_equal(ds.cpu().numpy(), os_)
    om = oracle_stores(k, pages, "k")[1]
    assert om[0, 0, 2, 4] == 60 and om[0, 0, 2, 5] == zc.RAW
    flags = om[..., 4:]
    assert 0 < np.mean(flags == zc.RAW) < 0.5  # the data has both kinds of chunk


def test_compress_open_page_into_its_slot():
    # a 16-row open-page buffer that has filled becomes page p of the store; other pages stay
    w, inp = case(lens=[40, 40])
    pages = w.seq_len // zc.PAGE
    for role in ("k", "v"):
        full_s, full_m = oracle_stores(inp[role], pages, role)
        s, m = device_stores(inp[role], pages, role)
        p = 7
        open_page = inp[role][:, :, 16 * p:16 * (p + 1)].copy()
        s[:, :, p].fill_(0xAB)
        m[:, :, p].fill_(0xAB)
        tq.zip_compress(dev_bf16(open_page), s, m, ROLE[role], src_page0=0, dst_page0=p)
        assert np.array_equal(s.cpu().numpy(), full_s)
        assert np.array_equal(m.cpu().numpy(), full_m)


def run_attention(w, inp, lens, n_splits, q_dtype=torch.bfloat16, tail="cache"):
    pages = w.seq_len // zc.PAGE
    ks, km = device_stores(inp["k"], pages, "k")
    vs, vm = device_stores(inp["v"], pages, "v")
    if tail == "cache":
        kt, vt = dev_bf16(inp["k"]), dev_bf16(inp["v"])
    else:
        # open-page buffers of 16 rows: token t at row t mod 16, stale rows elsewhere
        kt = torch.zeros((w.batch, w.n_kv_heads, 16, 128), dtype=torch.bfloat16, device="cuda")
        vt = torch.zeros_like(kt)
        for b, t in enumerate(lens):
            for i in range(16 * (t // 16), t):
                kt[b, :, i % 16] = dev_bf16(inp["k"][b, :, i])
                vt[b, :, i % 16] = dev_bf16(inp["v"][b, :, i])
    qb = dev_bf16(inp["q"])
    q = qb if q_dtype == torch.bfloat16 else qb.float().to(q_dtype)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    res = tq.zip_attention(ks, km, vs, vm, kt, vt, q, seq_lens=seq, max_len=max(lens), scale=w.scale,
                           n_splits=n_splits)
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in res]


def oracle_attention(w, inp, lens):
    pages = w.seq_len // zc.PAGE
    ks, km = oracle_stores(inp["k"], pages, "k")
    vs, vm = oracle_stores(inp["v"], pages, "v")
    return zc.decode_from_pages(inp["q"], ks, km, vs, vm, inp["k"], inp["v"], lens, w.scale)


def check_rows(out, lse, ref_o, ref_l, lens, g):
    for b, t in enumerate(lens):
        for h in range(out.shape[1]):
            if t == 0:
                assert lse[b, h] == -np.inf and not out[b, h].any()
                continue
            err = row_rel_err(out[b, h], ref_o[b, h])
            assert err <= RTOL, (b, h, err)
            assert abs(lse[b, h] - ref_l[b, h]) <= LSE_ATOL, (b, h)


@pytest.mark.parametrize("q_dtype", [torch.bfloat16, torch.float32, torch.float16])
def test_attention_matches_oracle(q_dtype):
    # fp32 and fp16 queries are the BF16 one converted: exact in fp32; in fp16 exact but for
    # components below fp16's normal range, which move by less than 2^-24
    w, inp = case()
    out, lse = run_attention(w, inp, LENS, 1, q_dtype)
    ref_o, ref_l = oracle_attention(w, inp, LENS)
    check_rows(out, lse, ref_o, ref_l, LENS, w.group_size)


@pytest.mark.parametrize("n_splits", [3, 40])
def test_sections_match_oracle_and_merge(n_splits):
    w, inp = case()
    po, pl = run_attention(w, inp, LENS, n_splits)
    pages = w.seq_len // zc.PAGE
    ks, km = oracle_stores(inp["k"], pages, "k")
    vs, vm = oracle_stores(inp["v"], pages, "v")
    q = zc.bf16_to_float(inp["q"])
    g = w.group_size
    for b, t in enumerate(LENS):
        kf = [zc.bf16_to_float(zc.row_tokens(ks[b, h], km[b, h], inp["k"][b, h], t, "k"))
              for h in range(w.n_kv_heads)]
        vf = [zc.bf16_to_float(zc.row_tokens(vs[b, h], vm[b, h], inp["v"][b, h], t, "v"))
              for h in range(w.n_kv_heads)]
        for s, (lo, hi) in enumerate(zc.section_bounds(t, n_splits)):
            for h in range(w.n_q_heads):
                ro, rl = attention.softmax_attend(q[b, h], kf[h // g][lo:hi], vf[h // g][lo:hi], w.scale)
                if hi == lo:
                    assert pl[s, b, h] == -np.inf and not po[s, b, h].any()
                else:
                    assert row_rel_err(po[s, b, h], ro) <= RTOL, (s, b, h)
                    assert abs(pl[s, b, h] - rl) <= LSE_ATOL
    # merging the sections (no rotation) gives the whole-row result
    out, lse = tq.merge_splits(None, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    ref_o, ref_l = oracle_attention(w, inp, LENS)
    check_rows(out.cpu().numpy(), lse.cpu().numpy(), ref_o, ref_l, LENS, g)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (16, 2), (32, 2)])
def test_head_groupings(hq, hkv):
    # one query head per KV head; 8 (one slice of 8 heads); 16 (two slices)
    lens = [309, 23]
    w, inp = case(hq=hq, hkv=hkv, lens=lens)
    for n_splits in (1, 5):
        if n_splits == 1:
            out, lse = run_attention(w, inp, lens, 1)
        else:
            po, pl = run_attention(w, inp, lens, n_splits)
            o, l_ = tq.merge_splits(None, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
            out, lse = o.cpu().numpy(), l_.cpu().numpy()
        ref_o, ref_l = oracle_attention(w, inp, lens)
        check_rows(out, lse, ref_o, ref_l, lens, w.group_size)


def test_open_page_buffer_equals_whole_cache_tail():
    w, inp = case()
    a = run_attention(w, inp, LENS, 1, tail="cache")
    b = run_attention(w, inp, LENS, 1, tail="open")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_merge_without_rotation_matches_oracle():
    rng = np.random.default_rng(3)
    s, bsz, hq = 7, 2, 8
    po = rng.standard_normal((s, bsz, hq, 128)).astype(np.float32)
    pl = (rng.standard_normal((s, bsz, hq)) * 3).astype(np.float32)
    pl[2, 0, :] = -np.inf
    pl[:, 1, 3] = -np.inf  # an empty row
    po[2, 0] = 0
    po[:, 1, 3] = 0
    out, lse = tq.merge_splits(None, torch.from_numpy(po).cuda(), torch.from_numpy(pl).cuda())
    ref_o, ref_l = attention.merge(po, pl)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    for b in range(bsz):
        for h in range(hq):
            if not np.isfinite(ref_l[b, h]):
                assert lse[b, h] == -np.inf and not out[b, h].any()
            else:
                assert row_rel_err(out[b, h], ref_o[b, h]) <= 1e-5
                assert abs(lse[b, h] - ref_l[b, h]) <= 1e-5

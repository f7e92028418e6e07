"""GPU parity of Block-GTQ keys through the C ABI against the oracle (oracle/blockgtq.py).

Encoding: codes equal the oracle's except coordinates whose rotated value lies within 1e-6
of a decision boundary (the library rotates with the fp32-rounded rotation, the oracle with
fp64: their rotated values differ by about 1e-7), at most 1e-5 of all coordinates (the
packed cache's code bar); norms within 1e-6 relative.  Attention is fed the oracle's codes and norms and compared with fp64
attention on the oracle's dequantised keys and the fp16 values: within 1e-4 relative per
row (fp32 sums of fp16 hi + lo operands), lse within 1e-4 + 1e-5 |lse|.  Rows are ragged, with an empty
one; sections 1, 3 and 40; query groups of 4, 8 and 16 heads (two slices).  Widths 1-4 (nibble
records of 64 bytes), 2-5 (80-byte records with a byte group) and 5-8 (128-byte records, byte
groups only).
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import row_rel_err
from oracle import attention, blockgtq as bg

pytestmark = pytest.mark.gpu

# fp16 operands with fp32 accumulation (the page's tensor-core form); keys, query and weights
# are each carried as fp16 hi + lo parts, so the sums keep fp32-level accuracy
RTOL = 1e-4
LSE_ATOL = 1e-4
LSE_RTOL = 1e-5
BOUNDARY_EPS = 1e-6
FLIP_FRACTION = 1e-5
LENS = [300, 77, 0]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


# (b_min, b_max, budget): nibble records; one byte group (80-byte records); byte groups only
RANGES = [(1, 4, 192), (2, 5, 192), (5, 8, 384)]


def case(hq=32, hkv=8, lens=LENS, cap=320, seed=0, widths=RANGES[0]):
    w = replace(workloads.WORKLOADS["gtq32k"], batch=len(lens), n_q_heads=hq, n_kv_heads=hkv, seq_len=cap)
    inp = workloads.generate(w, seed)
    s = bg.block_energies(inp["q_cal"], inp["k_cal"]).astype(np.float32)
    lo, hi, budget = widths
    bits = np.stack([bg.allocate(s[h].astype(np.float64), budget, lo, hi) for h in range(hkv)])
    enc = [bg.head_encoders(bits[h], inp["gauss"][h].astype(np.float64)) for h in range(hkv)]
    print("gtq case", (len(lens), hq, hkv, cap), "lens", lens, "seed", seed, "widths", widths, flush=True)
    return w, inp, bits, enc


def pack_records(oc, enc, cb):
    """The oracle's codes [b, kv, T, 128] as records of cb bytes, each head in its layout."""
    out = np.zeros(oc.shape[:3] + (cb,), np.uint8)
    for h in range(oc.shape[1]):
        out[:, h] = bg.pack_codes(oc[:, h].reshape(-1, 128), enc[h], record_bytes=cb).reshape(oc.shape[0], -1, cb)
    return out


def unpack_records(codes, enc):
    c = codes.cpu().numpy() if hasattr(codes, "cpu") else codes
    out = np.zeros(c.shape[:3] + (128,), np.uint8)
    for h in range(c.shape[1]):
        out[:, h] = bg.unpack_codes(c[:, h].reshape(-1, c.shape[3]), enc[h]).reshape(c.shape[0], -1, 128)
    return out


def oracle_keys(w, inp, enc):
    bsz, hkv, cap = w.batch, w.n_kv_heads, w.seq_len
    codes = np.zeros((bsz, hkv, cap, 128), np.uint8)
    norms = np.zeros((bsz, hkv, cap, 4), np.float32)
    ys = np.zeros((bsz, hkv, cap, 128))
    for b in range(bsz):
        for h in range(hkv):
            c, n, y = bg.quantize_keys(inp["k"][b, h].astype(np.float64), enc[h])
            codes[b, h], ys[b, h] = c, y
            norms[b, h, :, :n.shape[1]] = n
    return codes, norms, ys


@pytest.mark.parametrize("widths", RANGES)
def test_encoding_matches_oracle(widths):
    w, inp, bits, enc = case(widths=widths)
    keys = tq.GtqKeys(bits, inp["gauss"])
    cb = keys.code_bytes
    assert cb == max(bg.code_bytes(e) for e in enc) and (cb > 64) == (widths[1] > 4)
    codes = torch.full((w.batch, w.n_kv_heads, w.seq_len, cb), 0xA5, dtype=torch.uint8, device="cuda")
    norms = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, 4), dtype=torch.float32, device="cuda")
    x = torch.from_numpy(inp["k"]).cuda()
    # two calls: the first 100 tokens, then the rest at position 100
    tq.gtq_quantize_keys(keys, x[:, :, :100].contiguous(), codes, norms, pos0=0)
    tq.gtq_quantize_keys(keys, x[:, :, 100:].contiguous(), codes, norms, pos0=100)
    torch.cuda.synchronize()
    oc, on, oy = oracle_keys(w, inp, enc)
    raw = codes.cpu().numpy()
    for h in range(w.n_kv_heads):  # padding past the head's layout is written as zeros
        assert not raw[:, h, :, enc_used(enc[h]):].any()
    got = unpack_records(raw, enc)
    bad = got != oc
    print("code flips: %d of %d" % (bad.sum(), bad.size), flush=True)
    assert bad.mean() <= FLIP_FRACTION, bad.mean()
    for b, h, t, j in zip(*np.nonzero(bad)):
        ends = np.cumsum([len(e[1]) for e in enc[h]])
        m = enc[h][int(np.searchsorted(ends, j, side="right"))][4]  # the position's group boundaries
        assert np.min(np.abs(m - oy[b, h, t, j])) < BOUNDARY_EPS
    # norms of absent groups are 0 on both sides
    assert np.allclose(norms.cpu().numpy(), on, rtol=1e-6, atol=1e-30)


def enc_used(e):
    p = bg.nibble_positions(e)
    return p // 2 + 128 - p


def device_inputs(w, inp, oc, on, enc, cb=64):
    codes = torch.from_numpy(pack_records(oc, enc, cb)).cuda()
    norms = torch.from_numpy(on).cuda()
    v = torch.from_numpy(inp["v"].astype(np.float16)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16)).cuda()
    return codes, norms, v, q


def oracle_attention(w, inp, enc, oc, on, lens):
    kd = np.zeros((w.batch, w.n_kv_heads, w.seq_len, 128))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            kd[b, h] = bg.dequantize_keys(oc[b, h], on[b, h, :, :len(enc[h])].astype(np.float64), enc[h])
    return attention.decode(inp["q"].astype(np.float64), kd, inp["v"].astype(np.float16).astype(np.float64), lens,
                            w.scale), kd


def check(out, lse, ro, rl, lens):
    worst = worst_lse = 0.0
    for b, t in enumerate(lens):
        for h in range(out.shape[1]):
            if t == 0:
                assert lse[b, h] == -np.inf and not out[b, h].any()
                continue
            worst = max(worst, float(row_rel_err(out[b, h], ro[b, h])))
            worst_lse = max(worst_lse, abs(float(lse[b, h] - rl[b, h])))
    print("worst row error %.2e, lse %.2e" % (worst, worst_lse), flush=True)
    assert worst <= RTOL and worst_lse <= LSE_ATOL + LSE_RTOL * float(np.max(np.abs(rl[np.isfinite(rl)])))


@pytest.mark.parametrize("n_splits,widths", [(1, RANGES[0]), (3, RANGES[0]), (40, RANGES[0]), (1, RANGES[1]),
                                             (3, RANGES[2])])
def test_attention_matches_oracle(n_splits, widths):
    w, inp, bits, enc = case(widths=widths)
    keys = tq.GtqKeys(bits, inp["gauss"])
    oc, on, _ = oracle_keys(w, inp, enc)
    codes, norms, v, q = device_inputs(w, inp, oc, on, enc, keys.code_bytes)
    seq = torch.tensor(LENS, dtype=torch.int32, device="cuda")
    res = tq.gtq_attention(keys, codes, norms, v, q, seq_lens=seq, max_len=max(LENS), scale=w.scale, n_splits=n_splits)
    if n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    (ro, rl), _ = oracle_attention(w, inp, enc, oc, on, LENS)
    check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, LENS)


@pytest.mark.parametrize("hq,hkv", [(16, 2), (32, 2)])
def test_head_groupings(hq, hkv):
    lens = [300, 31]
    w, inp, bits, enc = case(hq=hq, hkv=hkv, lens=lens)
    keys = tq.GtqKeys(bits, inp["gauss"])
    oc, on, _ = oracle_keys(w, inp, enc)
    codes, norms, v, q = device_inputs(w, inp, oc, on, enc, keys.code_bytes)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out, lse = tq.gtq_attention(keys, codes, norms, v, q, seq_lens=seq, max_len=max(lens), scale=w.scale)
    torch.cuda.synchronize()
    (ro, rl), _ = oracle_attention(w, inp, enc, oc, on, lens)
    check(out.cpu().numpy(), lse.cpu().numpy(), ro, rl, lens)


def test_sections_are_the_oracle_splits():
    w, inp, bits, enc = case()
    keys = tq.GtqKeys(bits, inp["gauss"])
    oc, on, _ = oracle_keys(w, inp, enc)
    codes, norms, v, q = device_inputs(w, inp, oc, on, enc, keys.code_bytes)
    seq = torch.tensor(LENS, dtype=torch.int32, device="cuda")
    po, pl = tq.gtq_attention(keys, codes, norms, v, q, seq_lens=seq, max_len=max(LENS), scale=w.scale, n_splits=3)
    torch.cuda.synchronize()
    _, kd = oracle_attention(w, inp, enc, oc, on, LENS)
    ro, rl = attention.decode_splits(inp["q"].astype(np.float64), kd, inp["v"].astype(np.float16).astype(np.float64),
                                     LENS, w.scale, 3)
    po, pl = po.cpu().numpy(), pl.cpu().numpy()
    for s in range(3):
        for b, t in enumerate(LENS):
            for h in range(w.n_q_heads):
                if not np.isfinite(rl[s, b, h]):
                    assert pl[s, b, h] == -np.inf and not po[s, b, h].any()
                else:
                    assert row_rel_err(po[s, b, h], ro[s, b, h]) <= RTOL
                    assert abs(pl[s, b, h] - rl[s, b, h]) <= LSE_ATOL + LSE_RTOL * abs(rl[s, b, h])


# explicit allocations per KV head: one group (4 k-blocks), two groups of 64 (4 blocks),
# four groups with odd-sized tails (7 blocks), and three groups (5 blocks)
PATTERNS = [
    [3] * 64,
    [2] * 32 + [4] * 32,
    [1] * 3 + [2] * 20 + [3] * 20 + [4] * 21,
    [4, 1] * 8 + [3] * 48,
]


def test_allocation_shapes():
    lens = [300, 45]
    w, inp, _, _ = case(hq=16, hkv=4, lens=lens)
    bits = np.array(PATTERNS, dtype=np.int32)
    enc = [bg.head_encoders(bits[h], inp["gauss"][h].astype(np.float64)) for h in range(4)]
    keys = tq.GtqKeys(bits, inp["gauss"])
    assert [keys.n_groups(h) for h in range(4)] == [1, 2, 4, 3]
    oc, on, _ = oracle_keys(w, inp, enc)
    codes, norms, v, q = device_inputs(w, inp, oc, on, enc, keys.code_bytes)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for n_splits in (1, 3):
        res = tq.gtq_attention(keys, codes, norms, v, q, seq_lens=seq, max_len=max(lens), scale=w.scale,
                               n_splits=n_splits)
        if n_splits > 1:
            res = tq.merge_splits(None, *res)
        torch.cuda.synchronize()
        (ro, rl), _ = oracle_attention(w, inp, enc, oc, on, lens)
        check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, lens)


def device_cache(w, inp, keys):
    codes = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, keys.code_bytes), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((w.batch, w.n_kv_heads, w.seq_len, 4), dtype=torch.float32, device="cuda")
    tq.gtq_quantize_keys(keys, torch.from_numpy(inp["k"]).cuda(), codes, norms, pos0=0)
    v = torch.from_numpy(inp["v"].astype(np.float16)).cuda()
    return codes, norms, v


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("n_splits,widths", [(1, RANGES[0]), (3, RANGES[0]), (3, RANGES[1]), (1, RANGES[2])])
def test_append_step_equals_encode_then_attend(n_splits, widths):
    # one launch (encode the new key and write its value at slot P, then attend over P + 1
    # tokens) against the two calls it stands for: bit for bit, cache and outputs
    lens = [320, 320, 320]
    w, inp, bits, enc = case(lens=lens, widths=widths)
    keys = tq.GtqKeys(bits, inp["gauss"])
    P = 250
    rng = np.random.default_rng(7)
    k_new = torch.from_numpy((rng.standard_normal((3, w.n_kv_heads, 128)) * 3).astype(np.float16)).cuda()
    v_new = torch.from_numpy(rng.standard_normal((3, w.n_kv_heads, 128)).astype(np.float16)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16)).cuda()
    a = device_cache(w, inp, keys)
    b = tuple(t.clone() for t in a)
    res_a = tq.gtq_append_attention(keys, *a, k_new, v_new, q, pos0=P, scale=w.scale, n_splits=n_splits)
    tq.gtq_quantize_keys(keys, k_new[:, :, None, :].contiguous(), b[0], b[1], pos0=P)
    b[2][:, :, P] = v_new
    res_b = tq.gtq_attention(keys, *b, q, max_len=P + 1, scale=w.scale, n_splits=n_splits)
    torch.cuda.synchronize()
    assert same(a, b)
    assert same(res_a, res_b)


def test_append_step_per_row_slots():
    # device positions per row (a row of one token, a slot on a section boundary), fp32 new
    # tokens, and the new records against the oracle's encoding
    lens = [320, 320, 320, 320]
    w, inp, bits, enc = case(lens=lens)
    keys = tq.GtqKeys(bits, inp["gauss"])
    pos = [299, 0, 100, 33]
    rng = np.random.default_rng(8)
    kn = (rng.standard_normal((4, w.n_kv_heads, 128)) * 2).astype(np.float32)
    vn = rng.standard_normal((4, w.n_kv_heads, 128)).astype(np.float32)
    k_new, v_new = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float32)).cuda()
    pos_d = torch.tensor(pos, dtype=torch.int32, device="cuda")
    a = device_cache(w, inp, keys)
    b = tuple(t.clone() for t in a)
    res_a = tq.gtq_append_attention(keys, *a, k_new, v_new, q, pos=pos_d, scale=w.scale, n_splits=3)
    for r, p in enumerate(pos):
        tq.gtq_quantize_keys(keys, k_new[r:r + 1, :, None, :].contiguous(), b[0][r:r + 1], b[1][r:r + 1], pos0=p)
        b[2][r, :, p] = v_new[r].half()
    res_b = tq.gtq_attention(keys, *b, q, seq_lens=pos_d + 1, max_len=max(pos) + 1, scale=w.scale, n_splits=3)
    torch.cuda.synchronize()
    assert same(a, b)
    assert same(res_a, res_b)
    codes = unpack_records(a[0], enc)
    norms = a[1].cpu().numpy()
    for r, p in enumerate(pos):
        for h in range(w.n_kv_heads):
            oc, on, oy = bg.quantize_keys(kn[r, h][None].astype(np.float64), enc[h])
            bad = np.nonzero(codes[r, h, p] != oc[0])[0]
            assert len(bad) <= 2
            ends = np.cumsum([len(e[1]) for e in enc[h]])
            for j in bad:
                m = enc[h][int(np.searchsorted(ends, j, side="right"))][4]
                assert np.min(np.abs(m - oy[0, j])) < BOUNDARY_EPS
            assert np.allclose(norms[r, h, p, :len(enc[h])], on[0], rtol=1e-6)


def test_capacity_off_the_tile_grid():
    # a capacity that is not a multiple of 16: the last tile's copies past the capacity are
    # redirected inside the row, and the fused step appends at the last slot
    lens = [301, 17]
    w, inp, bits, enc = case(lens=lens, cap=301)
    keys = tq.GtqKeys(bits, inp["gauss"])
    oc, on, _ = oracle_keys(w, inp, enc)
    codes, norms, v, q = device_inputs(w, inp, oc, on, enc, keys.code_bytes)
    seq = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for n_splits in (1, 4):
        res = tq.gtq_attention(keys, codes, norms, v, q, seq_lens=seq, max_len=301, scale=w.scale, n_splits=n_splits)
        if n_splits > 1:
            res = tq.merge_splits(None, *res)
        torch.cuda.synchronize()
        (ro, rl), _ = oracle_attention(w, inp, enc, oc, on, lens)
        check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, lens)
    # the fused step at slot 300 (the capacity's last) against the two calls
    k_new = torch.from_numpy(inp["k"][:, :, 300].astype(np.float16)).cuda()
    v_new = torch.from_numpy(inp["v"][:, :, 300].astype(np.float16)).cuda()
    a = (codes.clone(), norms.clone(), v.clone())
    b = (codes.clone(), norms.clone(), v.clone())
    res_a = tq.gtq_append_attention(keys, *a, k_new, v_new, q, pos0=300, scale=w.scale, n_splits=4)
    tq.gtq_quantize_keys(keys, k_new[:, :, None, :].contiguous(), b[0], b[1], pos0=300)
    b[2][:, :, 300] = v_new
    res_b = tq.gtq_attention(keys, *b, q, max_len=301, scale=w.scale, n_splits=4)
    torch.cuda.synchronize()
    assert same(a, b) and same(res_a, res_b)

"""Parity at the benchmark sizes, in the launch configuration bench.py times, on sampled outputs.

Each test builds one benchmark workload at its full size (the packed-cache configurations:
isoquant32k B=8 T=32768 TQ3 with SO(4), long128k B=1 T=131072 with 64 sections, batched B=32
T=4096 TQ4/TQ3, gqa8k B=1 T=8192 with 32 sections, tiny T=256 fp32; zipfusion8k: B=32, T=8200, lossless BF16 pages; gtq32k: B=4, T=32768, Block-GTQ keys;
qjl32k: B=4, T=32768, two-stage keys with one-bit first-stage codes),
runs the step bench.py times (append of slot T-1 fused into the attention launch where the
format has one, the same sections, then the merge) and compares every query head of three
(sequence, KV head) units with the oracle, which encodes and attends over those units alone.
Bars: 2e-3 per row for the packed cache (fp16 weights, the tolerance of the other packed-cache
parity tests), 1e-4 for the lossless codec, Block-GTQ and two-stage keys (hi + lo fp16 operands).
One more case fills a stream of the largest capacity the library accepts (2^24 tokens) and
reads all of it.
"""

import time

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import OUT_RTOL, check_codes, dequantized, oracle_quantize, row_rel_err, unpack
from oracle import attention, blockgtq as bg, codebook, qjl, quant, zipcodec as zc

pytestmark = pytest.mark.gpu

EXACT_RTOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


def units(w):
    return [(0, 0), (w.batch // 2, min(w.n_kv_heads - 1, w.n_kv_heads // 2 + 1)), (w.batch - 1, w.n_kv_heads - 1)]


def announce(name, w):
    print("full-size case %s: B=%d Hq=%d Hkv=%d T=%d S=%d" % (name, w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len,
                                                              w.n_splits), flush=True)


@pytest.mark.parametrize("name", ["isoquant32k", "long128k", "batched", "gqa8k", "tiny"])
def test_packed_cache_step(name):
    # every packed-cache configuration at full size, with its own section count: isoquant32k
    # (whole-head rotation with SO(4)), long128k (64 key chunks and their merge), batched (TQ4
    # keys / TQ3 values, more workgroups than compute units), gqa8k (32 sections), tiny (fp32,
    # one section)
    w = workloads.WORKLOADS[name]
    announce(w.name, w)
    inp = workloads.generate(w, 0)
    T, S = w.seq_len, w.n_splits
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).cuda()
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, so4)
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    kc = tq.PackedCache(w.batch, w.n_kv_heads, T, w.bits_k, w.group, tq.TQ_KEYS)
    vc = tq.PackedCache(w.batch, w.n_kv_heads, T, w.bits_v, w.group, tq.TQ_VALUES)
    tq.quantize_append_kv(rot, kc, vc, kx[:, :, :T - 1].contiguous(), vx[:, :, :T - 1].contiguous())
    q = torch.from_numpy(inp["q"]).cuda()
    if S == 1:
        out, lse = tq.append_decode_attention(rot, kc, vc, kx[:, :, T - 1:].contiguous(), vx[:, :, T - 1:].contiguous(),
                                              q, pos0=T - 1, scale=w.scale, n_splits=1)
    else:
        po, pl = tq.append_decode_attention(rot, kc, vc, kx[:, :, T - 1:].contiguous(), vx[:, :, T - 1:].contiguous(),
                                            q, pos0=T - 1, scale=w.scale, n_splits=S)
        out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    del kx, vx, kc, vc
    ck, mk = codebook.lloyd_max(w.bits_k, w.group)
    cv, mv = codebook.lloyd_max(w.bits_v, w.group)
    worst, worst_lse, t0 = 0.0, 0.0, time.perf_counter()
    for b, kv in sorted(set(units(w))):
        so = None if inp["so4"] is None else inp["so4"][kv]
        sg = inp["signs"][kv]
        ki, kn, _ = quant.quantize(inp["k"][b, kv].astype(np.float64), sg, w.group, ck, mk, so)
        vi, vn, _ = quant.quantize(inp["v"][b, kv].astype(np.float64), sg, w.group, cv, mv, so)
        kd = quant.dequantize(ki, kn, sg, w.group, ck, so)
        vd = quant.dequantize(vi, vn, sg, w.group, cv, so)
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref, ref_lse = attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
            worst = max(worst, float(row_rel_err(out[b, h], ref)))
            worst_lse = max(worst_lse, abs(float(lse[b, h]) - ref_lse) / max(1.0, abs(ref_lse)))
    print("worst row error %.2e, lse %.2e (oracle %.1fs)" % (worst, worst_lse, time.perf_counter() - t0), flush=True)
    assert worst <= OUT_RTOL
    assert worst_lse <= 1e-4


def test_zipfusion8k_step():
    w = workloads.WORKLOADS["zipfusion8k"]
    announce(w.name, w)
    inp = workloads.generate(w, 0)
    T, pages = w.seq_len, w.seq_len // 16

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    stores, tails = [], []
    for role, rc in (("k", tq.TQ_KEYS), ("v", tq.TQ_VALUES)):
        s, m = tq.zip_store(w.batch, w.n_kv_heads, pages)
        tq.zip_compress(bf16(inp[role][:, :, :16 * pages]), s, m, rc, n_pages=pages)
        t = torch.zeros((w.batch, w.n_kv_heads, 16, 128), dtype=torch.bfloat16, device="cuda")
        t[:, :, :T - 16 * pages] = bf16(inp[role][:, :, 16 * pages:T])
        stores += [s, m]
        tails.append(t)
    res = tq.zip_attention(*stores, *tails, bf16(inp["q"]), max_len=T, scale=w.scale, n_splits=w.n_splits)
    if w.n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    out = res[0].cpu().numpy()
    worst = 0.0
    for b, kv in units(w):
        kf, vf = zc.bf16_to_float(inp["k"][b, kv, :T]), zc.bf16_to_float(inp["v"][b, kv, :T])
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref, _ = attention.softmax_attend(zc.bf16_to_float(inp["q"][b, h]), kf, vf, w.scale)
            worst = max(worst, float(row_rel_err(out[b, h], ref)))
    print("worst row error %.2e" % worst, flush=True)
    assert worst <= EXACT_RTOL


def test_gtq32k_step():
    w = workloads.WORKLOADS["gtq32k"]
    announce(w.name, w)
    inp = workloads.generate(w, 0)
    T, S = w.seq_len, w.n_splits
    energies = tq.gtq_block_energies(inp["q_cal"], inp["k_cal"])
    bits = np.stack([tq.gtq_allocate(energies[h], w.bits_k * 64, 1, 4) for h in range(w.n_kv_heads)])
    keys = tq.GtqKeys(bits, inp["gauss"])
    codes = torch.zeros((w.batch, w.n_kv_heads, T, keys.code_bytes), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((w.batch, w.n_kv_heads, T, 4), dtype=torch.float32, device="cuda")
    kx = torch.from_numpy(inp["k"]).cuda()
    v = torch.from_numpy(inp["v"]).cuda()
    tq.gtq_quantize_keys(keys, kx[:, :, :T - 1].contiguous(), codes, norms)
    q = torch.from_numpy(inp["q"]).cuda()
    po, pl = tq.gtq_append_attention(keys, codes, norms, v, kx[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous(),
                                     q, pos0=T - 1, scale=w.scale, n_splits=S)
    out, lse = tq.merge_splits(None, po, pl)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for b, kv in units(w):
        # the library's allocation is the oracle's (exact, checked on the CPU)
        enc = bg.head_encoders(bits[kv], inp["gauss"][kv].astype(np.float64))
        c, nrm, _ = bg.quantize_keys(inp["k"][b, kv].astype(np.float64), enc)
        kd = bg.dequantize_keys(c, nrm, enc)
        vd = inp["v"][b, kv].astype(np.float64)
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref, _ = attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
            worst = max(worst, float(row_rel_err(out[b, h], ref)))
    print("worst row error %.2e" % worst, flush=True)
    assert worst <= EXACT_RTOL


def test_qjl32k_step():
    w = workloads.WORKLOADS["qjl32k"]
    announce(w.name, w)
    inp = workloads.generate(w, 0)
    T, S = w.seq_len, w.n_splits
    keys = tq.QjlKeys(w.bits_k - 1, inp["gauss"], inp["proj"])
    codes = torch.zeros((w.batch, w.n_kv_heads, T, keys.code_bytes), dtype=torch.uint8, device="cuda")
    norms = torch.zeros((w.batch, w.n_kv_heads, T, 4), dtype=torch.float32, device="cuda")
    signs = torch.zeros((w.batch, w.n_kv_heads, T, 16), dtype=torch.uint8, device="cuda")
    kx = torch.from_numpy(inp["k"]).cuda()
    tq.qjl_quantize_keys(keys, kx[:, :, :T - 1].contiguous(), codes, norms, signs)
    v = torch.from_numpy(inp["v"]).cuda()
    q = torch.from_numpy(inp["q"]).cuda()
    # the step bench.py times: the new token's key and value written at slot T-1 inside the
    # attention launch
    po, pl = tq.qjl_append_attention(keys, codes, norms, signs, v, kx[:, :, T - 1].contiguous(),
                                     v[:, :, T - 1].contiguous(), q, pos0=T - 1, scale=w.scale, n_splits=S)
    out, lse = tq.merge_splits(None, po, pl)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for b, kv in units(w):
        enc = qjl.mse_encoders(w.bits_k - 1, inp["gauss"][kv].astype(np.float64))
        Sm = inp["proj"][kv].astype(np.float64)
        _, _, sg, rn, xh = qjl.encode_keys(inp["k"][b, kv].astype(np.float64), enc, Sm)
        vd = inp["v"][b, kv].astype(np.float64)
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref = qjl.attend(inp["q"][b, h].astype(np.float64), xh, sg, rn, Sm, vd, w.scale)
            worst = max(worst, float(row_rel_err(out[b, h], ref)))
    print("worst row error %.2e" % worst, flush=True)
    assert worst <= EXACT_RTOL


def test_maximum_capacity_step():
    # One (sequence, KV head) stream of TQ_MAX_CAPACITY tokens (IsoQuant TQ3 with SO(4), 4 query
    # heads): tile 0 takes 32 tokens and is copied to every tile but the last three; the last
    # 96 slots are written by one prefill call at cap - 96 (its two whole tiles on the matrix
    # cores, the partial last tile on the tile kernel) and by the step's fused append at
    # cap - 1, and the decode reads all 2^24 slots in 64 sections.  The oracle attends over
    # the 128 distinct tokens, the copied ones through the lse of their set plus the log of
    # their number of copies.
    from dataclasses import replace
    cap = tq.MAX_CAPACITY
    w = replace(workloads.WORKLOADS["isoquant32k"], batch=1, n_q_heads=4, n_kv_heads=1, seq_len=128, n_splits=64)
    announce("maximum capacity %d" % cap, w)
    inp = workloads.generate(w, 0)
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, torch.from_numpy(inp["so4"]).cuda())
    kx, vx = torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda()
    kc = tq.PackedCache(1, 1, cap, w.bits_k, w.group, tq.TQ_KEYS)
    vc = tq.PackedCache(1, 1, cap, w.bits_v, w.group, tq.TQ_VALUES)
    ntile = cap // tq.TILE
    tq.quantize_append_kv(rot, kc, vc, kx[:, :, :32].contiguous(), vx[:, :, :32].contiguous(), pos0=0)
    kt = kc.codes.view(1, 1, ntile, -1)
    for a in (kt, vc.codes, kc.norms, vc.norms):
        a[:, :, 1:ntile - 3] = a[:, :, :1]
    tq.quantize_append_kv(rot, kc, vc, kx[:, :, 32:127].contiguous(), vx[:, :, 32:127].contiguous(), pos0=cap - 96)
    q = torch.from_numpy(inp["q"]).cuda()
    po, pl = tq.append_decode_attention(rot, kc, vc, kx[:, :, 127:].contiguous(), vx[:, :, 127:].contiguous(), q,
                                        pos0=cap - 1, scale=w.scale, n_splits=w.n_splits)
    out, lse = tq.merge_splits(rot, po, pl)
    torch.cuda.synchronize()
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    # the cache's last three tiles and one copied tile in the middle, against the oracle
    oqk, oqv = oracle_quantize(w, inp, "k"), oracle_quantize(w, inp, "v")
    part = lambda oq, lo, hi: dict(oq, idx=oq["idx"][:, :, lo:hi], norms=oq["norms"][:, :, lo:hi],
                                   dist=oq["dist"][:, :, lo:hi])
    for tile, lo, n in ((ntile - 3, 32, 96), (ntile // 2, 0, 32)):
        nt = n // tq.TILE
        kcodes = kc.codes[:, :, tq.TILE * tile:tq.TILE * tile + n].cpu().numpy()
        vcodes = vc.codes[:, :, tile:tile + nt].cpu().numpy()
        for oq, codes, c, role in ((oqk, kcodes, kc, "k"), (oqv, vcodes, vc, "v")):
            idx, nrm = unpack(codes, c.norms[:, :, tile:tile + nt].cpu().numpy(), oq["bits"], role)
            check_codes(idx, nrm, part(oq, lo, lo + n), n)
    del kc, vc, kt
    kd, vd = dequantized(w, inp, oqk)[0, 0], dequantized(w, inp, oqv)[0, 0]
    copies = (cap - 96) // 32
    worst = worst_lse = 0.0
    for h in range(w.n_q_heads):
        qh = inp["q"][0, h].astype(np.float64)
        oa, la = attention.softmax_attend(qh, kd[:32], vd[:32], w.scale)
        ob, lb = attention.softmax_attend(qh, kd[32:], vd[32:], w.scale)
        ref, ref_lse = attention.merge(np.stack([oa, ob]), np.array([la + np.log(copies), lb]))
        worst = max(worst, float(row_rel_err(out[0, h], ref)))
        worst_lse = max(worst_lse, abs(float(lse[0, h]) - float(ref_lse)) / max(1.0, abs(float(ref_lse))))
    print("worst row error %.2e, lse %.2e" % (worst, worst_lse), flush=True)
    assert worst <= OUT_RTOL
    assert worst_lse <= 1e-4


def test_prefill_call_past_the_matrix_core_limit():
    # One call of 2^22 + 33 fp16 vectors per row (one sequence, one KV head, IsoQuant TQ3 with
    # SO(4)) at slot 7: calls longer than 2^22 vectors per row are taken whole by the
    # per-token kernel.  A seeded 4096-token block is repeated to that length; sampled slots
    # at the start, the middle and the end match the oracle's codes and norms.
    from dataclasses import replace
    n = (1 << 22) + 33
    pos0 = 7
    cap = (pos0 + n + tq.TILE - 1) // tq.TILE * tq.TILE
    w = replace(workloads.WORKLOADS["isoquant32k"], batch=1, n_q_heads=4, n_kv_heads=1, seq_len=4096)
    announce("prefill of %d tokens" % n, w)
    inp = workloads.generate(w, 3)
    reps = (n + 4095) // 4096
    kx = torch.from_numpy(inp["k"]).cuda().repeat(1, 1, reps, 1)[:, :, :n].contiguous()
    vx = torch.from_numpy(inp["v"]).cuda().repeat(1, 1, reps, 1)[:, :, :n].contiguous()
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, torch.from_numpy(inp["so4"]).cuda())
    kc = tq.PackedCache(1, 1, cap, w.bits_k, w.group, tq.TQ_KEYS)
    vc = tq.PackedCache(1, 1, cap, w.bits_v, w.group, tq.TQ_VALUES)
    tq.quantize_append_kv(rot, kc, vc, kx, vx, pos0=pos0)
    torch.cuda.synchronize()
    del kx, vx
    oqk, oqv = oracle_quantize(w, inp, "k"), oracle_quantize(w, inp, "v")
    part = lambda oq, idx: dict(oq, idx=oq["idx"][:, :, idx], norms=oq["norms"][:, :, idx], dist=oq["dist"][:, :, idx])
    ntile = cap // tq.TILE
    for tile in (0, 1, ntile // 2, ntile - 2, ntile - 1):
        slots = np.arange(tile * tq.TILE, (tile + 1) * tq.TILE)
        live = (slots >= pos0) & (slots < pos0 + n)
        src = (slots - pos0) % 4096  # the input token each slot holds
        kcodes = kc.codes[:, :, tile * tq.TILE:(tile + 1) * tq.TILE].cpu().numpy()
        vcodes = vc.codes[:, :, tile:tile + 1].cpu().numpy()
        for oq, codes, c, role in ((oqk, kcodes, kc, "k"), (oqv, vcodes, vc, "v")):
            idx, nrm = unpack(codes, c.norms[:, :, tile:tile + 1].cpu().numpy(), oq["bits"], role)
            check_codes(idx[:, :, live], nrm[:, :, live], part(oq, src[live]), int(live.sum()))
            assert not idx[:, :, ~live].any() and not nrm[:, :, ~live].any()  # slots outside the call

"""Benchmark: decode attention on a packed 3/4-bit KV cache, one MI355X.

One step = one pass of the whole hot path over one batch: quantise-append the newest
token's key and value into slot T-1 of every (sequence, KV head) and decode attention over
T tokens straight from the codes (rotated query, online softmax, rotated-domain value sum)
in one launch (tq_append_decode_attention: the workgroups whose key-axis section holds the
new slot write it first), then merge the key-axis splits with the single inverse rotation.  Inputs are seeded and
synthetic (workloads.py) and resident in HBM before timing.  The packed caches are
replicated to more than 1 GiB and cycled so that the 256 MB last-level cache cannot hold
them; the number is HBM-bound, not cache-bound.

Prints one JSON line.  Value = KV token*heads per second for the whole step.  The
roofline object is for that decode launch: algorithmic bytes (codes + norms of every
(token, KV head)) per launch over its average launch time, measured with events on the
launch stream.  cpu_baseline times the fp64 oracle (dequantise + plain attention) on a
bounded sample of the same workload on this host.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "decode attn KV token·heads/s + achieved HBM GB/s vs peak (TQ3, T=32K)"
HEADLINE = "isoquant32k"
HBM_PEAK_GBS = 8000.0
ZIP_RTOL = 1e-4  # lossless codec: fp32 sums of exact BF16 values against fp64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "compressed_domain_attention_amd", "csrc", "tq_kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


STEPS_PER_GRAPH = 8


def capture_graph(torch, fn, indices):
    """One HIP graph holding fn(i) for every i in indices (run once on a side stream first)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(indices[0])
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in indices:
            fn(i)
    return g


def time_steps(torch, step, reps, steps, warmup, check=None):
    """ms per step of `steps` steps that cycle through the reps cache replicas in order.  They
    run as replays of HIP graphs that each hold G consecutive steps (G the largest divisor of
    reps up to STEPS_PER_GRAPH, so the replicas keep their order), the remainder as one-step
    graphs: every step does its own GPU work, and the host's launch overhead is shared by G
    steps as it is by a model's layers.  Warm-up: at least `warmup` steps and 0.3 s, so the
    device is at its settled clock.  check() runs after the first replay and after the timed
    steps."""
    G = max(d for d in range(1, min(STEPS_PER_GRAPH, reps) + 1) if reps % d == 0)
    single = [capture_graph(torch, step, [r]) for r in range(reps)]
    multi = [capture_graph(torch, step, list(range(j * G, (j + 1) * G))) for j in range(reps // G)]
    single[0].replay()
    torch.cuda.synchronize()
    if check:
        check()
    t_w, i = time.perf_counter(), 0
    while i * G < warmup or time.perf_counter() - t_w < 0.3:
        multi[i % len(multi)].replay()
        i += 1
        if i % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    q, rem = divmod(steps, G)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(q):
        multi[i % len(multi)].replay()
    for i in range(rem):
        single[(q * G + i) % reps].replay()
    t1.record()
    torch.cuda.synchronize()
    if check:
        check()
    return t0.elapsed_time(t1) / steps


def bytes_per_token_head(w):
    """Packed bytes of one (token, KV head): key + value codes and fp32 group norms."""
    ng = 128 // w.group
    return (16 * w.bits_k + 4 * ng) + (16 * w.bits_v + 4 * ng)


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload, n_splits):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("kernel_sha256_16") != kernel_hash():
        return None
    ent = rec.get("workloads", {}).get("%s/S%d" % (workload, n_splits))
    return None if ent is None else ent["hbm_bytes_per_launch"]


def run_gpu(w, inp, steps, warmup, n_splits, schedule, check=True):
    import torch

    import compressed_domain_attention_amd as tq

    dev = torch.device("cuda:0")
    T = w.seq_len
    cap = (T + 31) // 32 * 32
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).to(dev)
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).to(dev), w.group, so4)
    q = torch.from_numpy(inp["q"]).to(dev)
    kx = torch.from_numpy(inp["k"]).to(dev)
    vx = torch.from_numpy(inp["v"]).to(dev)
    newk = kx[:, :, T - 1:T].contiguous()
    newv = vx[:, :, T - 1:T].contiguous()

    # prefill: the whole prompt (T - 1 tokens: slot T - 1 is the step's) quantised into both
    # caches in one launch, timed alone with events on the launch stream (the contiguous
    # prompt tensors exist before the timed region; one small call first loads the kernels)
    k0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev)
    v0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev)
    tq.quantize_append_kv(rot, k0, v0, newk, newv, pos0=0)
    pk = kx[:, :, :T - 1].contiguous() if T > 1 else kx
    pv = vx[:, :, :T - 1].contiguous() if T > 1 else vx
    del kx, vx
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    tq.quantize_append_kv(rot, k0, v0, pk, pv)
    e1.record()
    torch.cuda.synchronize()
    prefill_ms = e0.elapsed_time(e1)
    n_pre = pk.shape[2]
    in_bytes = 2 * n_pre * w.batch * w.n_kv_heads * 128 * pk.element_size()
    out_bytes = n_pre * w.batch * w.n_kv_heads * bytes_per_token_head(w)
    del pk, pv

    cache_bytes = sum(t.numel() * t.element_size() for t in (k0.codes, k0.norms, v0.codes, v0.norms))
    # replicas totalling >= 1 GiB defeat the 256 MB last-level cache (capped for tiny caches,
    # which then stay cache-resident: their number is a latency figure, not a bandwidth one)
    reps = min(256, max(2, math.ceil((1 << 30) / cache_bytes)))
    caches = [(k0, v0)]
    for _ in range(reps - 1):
        k = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev,
                           codes=k0.codes.clone(), norms=k0.norms.clone())
        v = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev,
                           codes=v0.codes.clone(), norms=v0.norms.clone())
        caches.append((k, v))
    log("cache %.1f MB x %d replicas" % (cache_bytes / 1e6, reps))
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    po = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads), dtype=torch.float32, device=dev)

    def decode(i):
        # the step's new key and value (slot T - 1) are quantised and written by the decode
        # launch itself, which then attends over all T tokens
        k, v = caches[i % reps]
        if n_splits == 1:
            tq.append_decode_attention(rot, k, v, newk, newv, q, pos0=T - 1, n_splits=1, schedule=schedule, out=out,
                                       lse=lse)
        else:
            tq.append_decode_attention(rot, k, v, newk, newv, q, pos0=T - 1, n_splits=n_splits, schedule=schedule,
                                       part_o=po, part_lse=pl)

    def step(i):
        decode(i)
        if n_splits > 1:
            tq.merge_splits(rot, po, pl, out=out, lse=lse)

    # eager warm-up, and the reference output that every graph replay must reproduce
    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    step(0)
    torch.cuda.synchronize()
    eager_out = out.clone()

    # the steps as HIP graph replays (no host work per kernel in the timed loop); every replay
    # must reproduce the eager step
    def same_as_eager():
        if not torch.equal(out, eager_out):
            raise SystemExit("graph replays do not reproduce the eager step")

    total_ms = steps * time_steps(torch, step, reps, steps, warmup, same_as_eager)
    # one graph holding a run of decode launches for the kernel timing
    n_dec = max(reps, 16)
    gdec = capture_graph(torch, decode, list(range(n_dec)))
    torch.cuda.synchronize()

    # decode kernel alone: back-to-back launches in one graph, events on the launch stream
    gdec.replay()
    torch.cuda.synchronize()
    t_d = time.perf_counter()
    gdec.replay()
    torch.cuda.synchronize()
    # about half a second of launches
    reps_dec = max(3, int(0.5 / max(time.perf_counter() - t_d, 1e-6)))
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(reps_dec):
        gdec.replay()
    d1.record()
    torch.cuda.synchronize()
    dec_ms = d0.elapsed_time(d1) / (reps_dec * n_dec)

    parity = None
    if check:
        parity = sampled_parity(w, inp, out.cpu().numpy())
    return dict(ms_per_step=total_ms / steps, decode_ms=dec_ms, prefill_ms=prefill_ms, prefill_bytes=in_bytes + out_bytes,
                reps=reps, cache_bytes=cache_bytes, parity=parity, decode_launches=reps_dec * n_dec)


def run_tail(w, inp, n_tail, tail_splits, steps, warmup, n_splits, schedule):
    """The step with an unquantised tail of n_tail tokens per row (the pages' fp16 prefill or
    recent-token window): the packed append+decode launch into sections 0..S-1, dense attention
    over the tail into the next tail_splits sections, one merge over all of them.  The tail is
    the workload's first n_tail key/value vectors in its own dtype."""
    import torch

    import compressed_domain_attention_amd as tq
    from oracle import attention, codebook, quant

    dev = torch.device("cuda:0")
    T = w.seq_len
    cap = (T + 31) // 32 * 32
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).to(dev)
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).to(dev), w.group, so4)
    q = torch.from_numpy(inp["q"]).to(dev)
    k0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev)
    v0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev)
    tq.quantize_append(rot, k0, torch.from_numpy(inp["k"]).to(dev))
    tq.quantize_append(rot, v0, torch.from_numpy(inp["v"]).to(dev))
    newk = torch.from_numpy(inp["k"][:, :, T - 1:T].copy()).to(dev)
    newv = torch.from_numpy(inp["v"][:, :, T - 1:T].copy()).to(dev)
    kt = torch.from_numpy(inp["k"][:, :, :n_tail].copy()).to(dev)
    vt = torch.from_numpy(inp["v"][:, :, :n_tail].copy()).to(dev)
    cache_bytes = sum(t.numel() * t.element_size() for t in (k0.codes, k0.norms, v0.codes, v0.norms))
    reps = min(256, max(2, math.ceil((1 << 30) / cache_bytes)))
    caches = [(k0, v0)] + [
        (tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev, codes=k0.codes.clone(),
                        norms=k0.norms.clone()),
         tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev, codes=v0.codes.clone(),
                        norms=v0.norms.clone())) for _ in range(reps - 1)]
    S, St = n_splits, tail_splits
    po = torch.empty((S + St, w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((S + St, w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)

    def dense(i):
        tq.dense_attention(rot, kt, vt, q, max_len=n_tail, n_splits=St, part_o=po[S:], part_lse=pl[S:])

    def step(i):
        k, v = caches[i % reps]
        tq.append_decode_attention(rot, k, v, newk, newv, q, pos0=T - 1, n_splits=S, schedule=schedule,
                                   part_o=po[:S], part_lse=pl[:S])
        dense(i)
        tq.merge_splits(rot, po, pl, out=out, lse=lse)

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    step_ms = time_steps(torch, step, reps, steps, warmup)
    gd = capture_graph(torch, dense, list(range(16)))
    gd.replay()
    torch.cuda.synchronize()
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_d = time.perf_counter()
    n_rep = 0
    d0.record()
    while time.perf_counter() - t_d < 0.5:
        gd.replay()
        n_rep += 1
        if n_rep % 64 == 0:
            torch.cuda.synchronize()
    d1.record()
    torch.cuda.synchronize()
    dense_ms = d0.elapsed_time(d1) / (16 * n_rep)

    # sampled parity: two (sequence, KV head) units against the oracle over packed + tail
    from helpers import OUT_RTOL, row_rel_err
    o = out.cpu().numpy()
    worst = 0.0
    ck, mk = codebook.lloyd_max(w.bits_k, w.group)
    cv, mv = codebook.lloyd_max(w.bits_v, w.group)
    for b, kv in [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]:
        so = None if inp["so4"] is None else inp["so4"][kv]
        sg = inp["signs"][kv]
        ki, kn, _ = quant.quantize(inp["k"][b, kv].astype(np.float64), sg, w.group, ck, mk, so)
        vi, vn, _ = quant.quantize(inp["v"][b, kv].astype(np.float64), sg, w.group, cv, mv, so)
        kd = np.concatenate([quant.dequantize(ki, kn, sg, w.group, ck, so), inp["k"][b, kv, :n_tail]])
        vd = np.concatenate([quant.dequantize(vi, vn, sg, w.group, cv, so), inp["v"][b, kv, :n_tail]])
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref, _ = attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
            worst = max(worst, float(row_rel_err(o[b, h], ref)))
    if worst > OUT_RTOL:
        raise SystemExit("parity check failed: %.3e > %.1e" % (worst, OUT_RTOL))
    tail_bytes = 2 * w.batch * w.n_kv_heads * n_tail * 128 * kt.element_size()
    return dict(step_ms=step_ms, dense_ms=dense_ms, tail_bytes=tail_bytes, parity=worst, reps=reps)


ZIP_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "zip_traffic.json")
ZIP_KERNEL_SRC = os.path.join(ROOT, "compressed_domain_attention_amd", "csrc", "tq_zip.hip")


def zip_kernel_hash():
    return hashlib.sha256(open(ZIP_KERNEL_SRC, "rb").read()).hexdigest()[:16]


def zip_setup(w, inp, dev):
    """Compressed stores of the workload's K and V (every whole page of the row) plus the
    open-page buffers of 16 rows holding its last T mod 16 tokens, and the query."""
    import torch

    import compressed_domain_attention_amd as tq
    T = w.seq_len
    pages = T // 16

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    stores, compress_ms = [], []
    for role, rc in (("k", tq.TQ_KEYS), ("v", tq.TQ_VALUES)):
        x = bf16(inp[role][:, :, :16 * pages])
        s, m = tq.zip_store(w.batch, w.n_kv_heads, pages, device=dev)
        tq.zip_compress(x, s, m, rc, n_pages=1)  # loads the kernel before timing
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.zip_compress(x, s, m, rc, n_pages=pages)
        e1.record()
        torch.cuda.synchronize()
        compress_ms.append(e0.elapsed_time(e1))
        stores += [s, m]
        del x
    tails = []
    for role in ("k", "v"):
        t = torch.zeros((w.batch, w.n_kv_heads, 16, 128), dtype=torch.bfloat16, device=dev)
        n = T - 16 * pages
        if n:
            t[:, :, :n] = bf16(inp[role][:, :, 16 * pages:T])
        tails.append(t)
    q = bf16(inp["q"])
    return stores, tails, q, sum(compress_ms)


def zip_algorithmic_bytes(w, k_meta, v_meta):
    """KV bytes one launch must read: every page's stored chunks (768 coded, 1024 kept) and
    its 8 metadata bytes, and the open page's BF16 tokens, for keys and values."""
    total = 0
    for m in (k_meta, v_meta):
        flags = m[..., 4:].cpu().numpy()
        total += int(np.where(flags == 0xFF, 1024, 768).sum()) + 8 * flags.shape[0] * flags.shape[1] * flags.shape[2]
    total += 2 * w.batch * w.n_kv_heads * (w.seq_len % 16) * 256
    return total


def run_zip(w, inp, steps, warmup, n_splits, check=True):
    """The step on the lossless BF16 codec: attention read straight from the compressed
    pages (and the open page), its sections merged without rotation."""
    import torch

    import compressed_domain_attention_amd as tq

    dev = torch.device("cuda:0")
    (ks, km, vs, vm), (kt, vt), q, compress_ms = zip_setup(w, inp, dev)
    store_bytes = 2 * (ks.numel() + km.numel())
    reps = min(256, max(2, math.ceil((1 << 30) / store_bytes)))
    sets = [(ks, km, vs, vm)] + [tuple(t.clone() for t in (ks, km, vs, vm)) for _ in range(reps - 1)]
    log("compressed stores %.1f MB x %d replicas" % (store_bytes / 1e6, reps))
    S = n_splits
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    po = torch.empty((S, w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((S, w.batch, w.n_q_heads), dtype=torch.float32, device=dev)

    def attend(i):
        a = sets[i % reps]
        if S == 1:
            tq.zip_attention(*a, kt, vt, q, max_len=w.seq_len, scale=w.scale, out=out, lse=lse)
        else:
            tq.zip_attention(*a, kt, vt, q, max_len=w.seq_len, scale=w.scale, n_splits=S, part_o=po, part_lse=pl)

    def step(i):
        attend(i)
        if S > 1:
            tq.merge_splits(None, po, pl, out=out, lse=lse)

    def graph(fn, n):
        return capture_graph(torch, fn, list(range(n)))

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    eager_out = out.clone()

    def same_as_eager():
        if not torch.equal(out, eager_out):
            raise SystemExit("graph replays do not reproduce the eager step")

    step_ms = time_steps(torch, step, reps, steps, warmup, same_as_eager)
    n_att = max(reps, 16)
    ga = graph(lambda i: attend(i), n_att)
    ga.replay()
    torch.cuda.synchronize()
    t_d = time.perf_counter()
    ga.replay()
    torch.cuda.synchronize()
    reps_att = max(3, int(0.5 / max(time.perf_counter() - t_d, 1e-6)))
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(reps_att):
        ga.replay()
    d1.record()
    torch.cuda.synchronize()
    att_ms = d0.elapsed_time(d1) / (reps_att * n_att)

    parity = None
    if check:
        # lossless: the output must be attention on the original BF16 values
        from helpers import row_rel_err
        from oracle import attention, zipcodec as zc
        o = out.cpu().numpy()
        parity = 0.0
        for b, kv in [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]:
            kf = zc.bf16_to_float(inp["k"][b, kv, :w.seq_len])
            vf = zc.bf16_to_float(inp["v"][b, kv, :w.seq_len])
            for h in range(kv * w.group_size, (kv + 1) * w.group_size):
                ref, _ = attention.softmax_attend(zc.bf16_to_float(inp["q"][b, h]), kf, vf, w.scale)
                parity = max(parity, float(row_rel_err(o[b, h], ref)))
        if parity > ZIP_RTOL:
            raise SystemExit("parity check failed: %.3e > %.1e" % (parity, ZIP_RTOL))
    algo = zip_algorithmic_bytes(w, km, vm)
    raw = 2 * w.batch * w.n_kv_heads * w.seq_len * 256
    frac_kept = float(np.mean(np.concatenate([(m[..., 4:].cpu().numpy() == 0xFF).ravel() for m in (km, vm)])))
    return dict(step_ms=step_ms, attn_ms=att_ms, algo_bytes=algo, bf16_bytes=raw, reps=reps, parity=parity,
                compress_ms=compress_ms, kept_fraction=frac_kept, store_bytes=store_bytes)


def zip_counter_run(w, inp, n_splits, launches=24):
    """rocprofv3 --pmc dispatches for the codec: the calibration copies, then `launches`
    attention launches over the store replicas, as run_zip times them."""
    import ctypes

    import torch

    import compressed_domain_attention_amd as tq
    from compressed_domain_attention_amd import build as _b

    dev = torch.device("cuda:0")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.tq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.tq_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, 4096, stream) == 0
    torch.cuda.synchronize()
    del src, dst
    (ks, km, vs, vm), (kt, vt), q, _ = zip_setup(w, inp, dev)
    store_bytes = 2 * (ks.numel() + km.numel())
    reps = min(256, max(2, math.ceil((1 << 30) / store_bytes)))
    sets = [(ks, km, vs, vm)] + [tuple(t.clone() for t in (ks, km, vs, vm)) for _ in range(reps - 1)]
    po = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    for i in range(launches):
        a = sets[i % reps]
        if n_splits == 1:
            tq.zip_attention(*a, kt, vt, q, max_len=w.seq_len, scale=w.scale, out=out)
        else:
            tq.zip_attention(*a, kt, vt, q, max_len=w.seq_len, scale=w.scale, n_splits=n_splits, part_o=po,
                             part_lse=pl)
    torch.cuda.synchronize()
    log("counter run: 3 copies of %d bytes, %d zip attention launches over %d replicas" % (
        COPY_BYTES, launches, reps))


def zip_measured_traffic(workload, n_splits):
    if not os.path.exists(ZIP_TRAFFIC_FILE):
        return None
    rec = json.load(open(ZIP_TRAFFIC_FILE))
    if rec.get("kernel_sha256_16") != zip_kernel_hash():
        return None
    ent = rec.get("workloads", {}).get("%s/S%d" % (workload, n_splits))
    return None if ent is None else ent["hbm_bytes_per_launch"]


def gtq_setup(w, inp, dev):
    """Block-GTQ keys from the workload's calibration prefix (energies, allocation and
    encoders in the library), the prompt's keys encoded on the GPU (timed), fp16 values.
    The last token (slot T - 1) is the step's new one: its key and value are returned for
    the step to append."""
    import torch

    import compressed_domain_attention_amd as tq
    T = w.seq_len
    norms = torch.zeros((w.batch, w.n_kv_heads, T, 4), dtype=torch.float32, device=dev)
    x = torch.from_numpy(inp["k"]).to(dev)
    if w.codec == "qjl":  # two-stage keys
        bits = np.full((w.n_kv_heads, 64), w.bits_k - 1, dtype=np.int32)
        keys = tq.QjlKeys(w.bits_k - 1, inp["gauss"], inp["proj"], device=dev)
        codes = torch.zeros((w.batch, w.n_kv_heads, T, keys.code_bytes), dtype=torch.uint8, device=dev)
        signs = torch.zeros((w.batch, w.n_kv_heads, T, 16), dtype=torch.uint8, device=dev)
        prompt = x[:, :, :T - 1].contiguous()
        tq.qjl_quantize_keys(keys, prompt[:, :, :1].contiguous(), codes, norms, signs)  # loads the kernel
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        tq.qjl_quantize_keys(keys, prompt, codes, norms, signs)
        e1.record()
        torch.cuda.synchronize()
        v = torch.from_numpy(inp["v"]).to(dev)
        q = torch.from_numpy(inp["q"]).to(dev)
        k_new, v_new = x[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous()
        return keys, bits, codes, norms, v, q, k_new, v_new, e0.elapsed_time(e1), signs
    energies = tq.gtq_block_energies(inp["q_cal"], inp["k_cal"])
    bits = np.stack([tq.gtq_allocate(energies[h], w.bits_k * 64, *GTQ_RANGE) for h in range(w.n_kv_heads)])
    keys = tq.GtqKeys(bits, inp["gauss"], device=dev)
    codes = torch.zeros((w.batch, w.n_kv_heads, T, keys.code_bytes), dtype=torch.uint8, device=dev)
    prompt = x[:, :, :T - 1].contiguous()
    tq.gtq_quantize_keys(keys, prompt[:, :, :1].contiguous(), codes, norms)  # loads the kernel before timing
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    tq.gtq_quantize_keys(keys, prompt, codes, norms)
    e1.record()
    torch.cuda.synchronize()
    v = torch.from_numpy(inp["v"]).to(dev)
    q = torch.from_numpy(inp["q"]).to(dev)
    k_new, v_new = x[:, :, T - 1].contiguous(), v[:, :, T - 1].contiguous()
    return keys, bits, codes, norms, v, q, k_new, v_new, e0.elapsed_time(e1), None


# Block-GTQ widths [b_min, b_max] of the allocation (--gtq-widths); above 4 bits the
# high-bit groups take byte containers and the records grow past 64 bytes
GTQ_RANGE = (1, 4)


def gtq_bytes_per_token_head(code_bytes):
    return code_bytes + 16 + 256  # key codes, the four group norms, fp16 values
# two-stage keys: first-stage codes (b - 1 bits per coordinate, bit-packed), the norm
# slots, the residual's 128 sign bits, fp16 values
def qjl_bytes_per_token_head(w):
    return 16 * (w.bits_k - 1) + 16 + 16 + 256


def run_gtq(w, inp, steps, warmup, n_splits, check=True):
    """The step on Block-GTQ keys with fp16 values: one launch that appends the new token
    (key encoded, value written at slot T - 1) and attends over the T tokens in sections,
    then the merge without rotation."""
    import torch

    import compressed_domain_attention_amd as tq

    dev = torch.device("cuda:0")
    keys, bits, codes, norms, v, q, k_new, v_new, enc_ms, signs = gtq_setup(w, inp, dev)
    qjl = signs is not None
    cache = (codes, norms, v, signs) if qjl else (codes, norms, v)
    cache_bytes = sum(t.numel() * t.element_size() for t in cache)
    reps = min(256, max(2, math.ceil((1 << 30) / cache_bytes)))
    sets = [cache] + [tuple(t.clone() for t in cache) for _ in range(reps - 1)]
    log("cache %.1f MB x %d replicas; groups per head %s" % (cache_bytes / 1e6, reps,
                                                             [keys.n_groups(h) for h in range(w.n_kv_heads)]))
    S = n_splits
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    po = torch.empty((S, w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((S, w.batch, w.n_q_heads), dtype=torch.float32, device=dev)

    def attend(i):
        if qjl:
            c, n, vv, sg = sets[i % reps]
            if S == 1:
                tq.qjl_append_attention(keys, c, n, sg, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale,
                                        out=out, lse=lse)
            else:
                tq.qjl_append_attention(keys, c, n, sg, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale,
                                        n_splits=S, part_o=po, part_lse=pl)
            return
        c, n, vv = sets[i % reps]
        if S == 1:
            tq.gtq_append_attention(keys, c, n, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale, out=out,
                                    lse=lse)
        else:
            tq.gtq_append_attention(keys, c, n, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale, n_splits=S,
                                    part_o=po, part_lse=pl)

    def step(i):
        attend(i)
        if S > 1:
            tq.merge_splits(None, po, pl, out=out, lse=lse)

    def graph(fn, n):
        return capture_graph(torch, fn, list(range(n)))

    for i in range(max(warmup, 1)):
        step(i)
    torch.cuda.synchronize()
    eager_out = out.clone()

    def same_as_eager():
        if not torch.equal(out, eager_out):
            raise SystemExit("graph replays do not reproduce the eager step")

    step_ms = time_steps(torch, step, reps, steps, warmup, same_as_eager)
    n_att = max(reps, 16)
    ga = graph(lambda i: attend(i), n_att)
    ga.replay()
    torch.cuda.synchronize()
    t_d = time.perf_counter()
    ga.replay()
    torch.cuda.synchronize()
    reps_att = max(3, int(0.5 / max(time.perf_counter() - t_d, 1e-6)))
    d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    d0.record()
    for _ in range(reps_att):
        ga.replay()
    d1.record()
    torch.cuda.synchronize()
    att_ms = d0.elapsed_time(d1) / (reps_att * n_att)

    parity = None
    if check:
        # two (sequence, KV head) units against the oracle's own encoding of the same keys
        from helpers import OUT_RTOL, row_rel_err
        from oracle import attention, blockgtq as bg, qjl as oq
        o = out.cpu().numpy()
        parity = 0.0
        for b, kv in [(0, 0), (w.batch - 1, w.n_kv_heads - 1)] if qjl else []:
            enc = oq.mse_encoders(w.bits_k - 1, inp["gauss"][kv].astype(np.float64))
            S_ = inp["proj"][kv].astype(np.float64)
            _, _, sg, rn, xh = oq.encode_keys(inp["k"][b, kv].astype(np.float64), enc, S_)
            vd = inp["v"][b, kv].astype(np.float64)
            for h in range(kv * w.group_size, (kv + 1) * w.group_size):
                ref = oq.attend(inp["q"][b, h].astype(np.float64), xh, sg, rn, S_, vd, w.scale)
                parity = max(parity, float(row_rel_err(o[b, h], ref)))
        s = None if qjl else bg.block_energies(inp["q_cal"], inp["k_cal"]).astype(np.float32)
        for b, kv in [] if qjl else [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]:
            enc = bg.head_encoders(bg.allocate(s[kv].astype(np.float64), w.bits_k * 64, *GTQ_RANGE),
                                   inp["gauss"][kv].astype(np.float64))
            c, nrm, _ = bg.quantize_keys(inp["k"][b, kv].astype(np.float64), enc)
            kd = bg.dequantize_keys(c, nrm, enc)
            vd = inp["v"][b, kv].astype(np.float64)
            for h in range(kv * w.group_size, (kv + 1) * w.group_size):
                ref, _ = attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
                parity = max(parity, float(row_rel_err(o[b, h], ref)))
        if parity > OUT_RTOL:
            raise SystemExit("parity check failed: %.3e > %.1e" % (parity, OUT_RTOL))
    algo = w.batch * w.n_kv_heads * w.seq_len * (qjl_bytes_per_token_head(w) if qjl else
                                                 gtq_bytes_per_token_head(keys.code_bytes))
    return dict(step_ms=step_ms, attn_ms=att_ms, algo_bytes=algo, reps=reps, parity=parity, encode_ms=enc_ms,
                widths=np.bincount(bits.ravel(), minlength=9)[1:].tolist(), code_bytes=keys.code_bytes)


GTQ_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gtq_traffic.json")
GTQ_KERNEL_SRC = os.path.join(ROOT, "compressed_domain_attention_amd", "csrc", "tq_gtq.hip")


def gtq_kernel_hash():
    return hashlib.sha256(open(GTQ_KERNEL_SRC, "rb").read()).hexdigest()[:16]


def gtq_counter_run(w, inp, n_splits, launches=24):
    """rocprofv3 --pmc dispatches for Block-GTQ: the calibration copies, then `launches`
    append + attention launches over the cache replicas, as run_gtq times them."""
    import ctypes

    import torch

    import compressed_domain_attention_amd as tq
    from compressed_domain_attention_amd import build as _b

    dev = torch.device("cuda:0")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.tq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.tq_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, 4096, stream) == 0
    torch.cuda.synchronize()
    del src, dst
    keys, bits, codes, norms, v, q, k_new, v_new, _, signs = gtq_setup(w, inp, dev)
    cache = (codes, norms, v) if signs is None else (codes, norms, v, signs)
    cache_bytes = sum(t.numel() * t.element_size() for t in cache)
    reps = min(256, max(2, math.ceil((1 << 30) / cache_bytes)))
    sets = [cache] + [tuple(t.clone() for t in cache) for _ in range(reps - 1)]
    S = max(n_splits, 1)
    po = torch.empty((S, w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((S, w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    for i in range(launches):
        if signs is not None:
            c, n, vv, sg = sets[i % reps]
            if n_splits == 1:
                tq.qjl_append_attention(keys, c, n, sg, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale,
                                        out=out)
            else:
                tq.qjl_append_attention(keys, c, n, sg, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale,
                                        n_splits=n_splits, part_o=po, part_lse=pl)
            continue
        c, n, vv = sets[i % reps]
        if n_splits == 1:
            tq.gtq_append_attention(keys, c, n, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale, out=out)
        else:
            tq.gtq_append_attention(keys, c, n, vv, k_new, v_new, q, pos0=w.seq_len - 1, scale=w.scale,
                                    n_splits=n_splits, part_o=po, part_lse=pl)
    torch.cuda.synchronize()
    log("counter run: 3 copies of %d bytes, %d Block-GTQ attention launches over %d replicas" % (
        COPY_BYTES, launches, reps))


def gtq_measured_traffic(workload, n_splits):
    if not os.path.exists(GTQ_TRAFFIC_FILE):
        return None
    rec = json.load(open(GTQ_TRAFFIC_FILE))
    if rec.get("kernel_sha256_16") != gtq_kernel_hash():
        return None
    ent = rec.get("workloads", {}).get("%s/S%d" % (workload, n_splits))
    return None if ent is None else ent["hbm_bytes_per_launch"]


def _oracle_gtq_unit(args):
    w, b, kv = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import attention, blockgtq as bg
    inp = _oracle_unit.inp
    s = bg.block_energies(inp["q_cal"], inp["k_cal"]).astype(np.float32)
    enc = bg.head_encoders(bg.allocate(s[kv].astype(np.float64), w.bits_k * 64, *GTQ_RANGE),
                           inp["gauss"][kv].astype(np.float64))
    c, nrm, _ = bg.quantize_keys(inp["k"][b, kv].astype(np.float64), enc)  # the stored cache (not timed)
    t0 = time.perf_counter()
    kd = bg.dequantize_keys(c, nrm, enc)
    vd = inp["v"][b, kv].astype(np.float64)
    for h in range(kv * w.group_size, (kv + 1) * w.group_size):
        attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
    return time.perf_counter() - t0


def _oracle_qjl_unit(args):
    w, b, kv = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import qjl
    inp = _oracle_unit.inp
    enc = qjl.mse_encoders(w.bits_k - 1, inp["gauss"][kv].astype(np.float64))
    S = inp["proj"][kv].astype(np.float64)
    _, _, sg, rn, xh = qjl.encode_keys(inp["k"][b, kv].astype(np.float64), enc, S)  # the stored cache (not timed)
    t0 = time.perf_counter()
    vd = inp["v"][b, kv].astype(np.float64)
    for h in range(kv * w.group_size, (kv + 1) * w.group_size):
        qjl.attend(inp["q"][b, h].astype(np.float64), xh, sg, rn, S, vd, w.scale)
    return time.perf_counter() - t0


def _oracle_zip_unit(args):
    w, b, kv = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import attention, zipcodec as zc
    inp = _oracle_unit.inp
    T = w.seq_len
    pages = T // zc.PAGE
    ks, km = zc.compress_stream(inp["k"][b, kv], pages, "k")  # the cache as stored (not timed)
    vs, vm = zc.compress_stream(inp["v"][b, kv], pages, "v")
    t0 = time.perf_counter()
    kf = zc.bf16_to_float(zc.row_tokens(ks, km, inp["k"][b, kv], T, "k"))
    vf = zc.bf16_to_float(zc.row_tokens(vs, vm, inp["v"][b, kv], T, "v"))
    for h in range(kv * w.group_size, (kv + 1) * w.group_size):
        attention.softmax_attend(zc.bf16_to_float(inp["q"][b, h]), kf, vf, w.scale)
    return time.perf_counter() - t0


def sampled_parity(w, inp, out):
    """Oracle check of a few (sequence, query head) rows of the measured output."""
    from helpers import OUT_RTOL, row_rel_err
    from oracle import attention, codebook, quant

    t0 = time.perf_counter()
    worst = 0.0
    units = [(0, 0), (w.batch - 1, w.n_kv_heads - 1)]
    ck, mk = codebook.lloyd_max(w.bits_k, w.group)
    cv, mv = codebook.lloyd_max(w.bits_v, w.group)
    for b, kv in units:
        so = None if inp["so4"] is None else inp["so4"][kv]
        sg = inp["signs"][kv]
        ki, kn, _ = quant.quantize(inp["k"][b, kv].astype(np.float64), sg, w.group, ck, mk, so)
        vi, vn, _ = quant.quantize(inp["v"][b, kv].astype(np.float64), sg, w.group, cv, mv, so)
        kd = quant.dequantize(ki, kn, sg, w.group, ck, so)
        vd = quant.dequantize(vi, vn, sg, w.group, cv, so)
        for h in range(kv * w.group_size, (kv + 1) * w.group_size):
            ref, _ = attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
            worst = max(worst, float(row_rel_err(out[b, h], ref)))
    log("sampled parity: worst row rel err %.3e over %d heads (%.1fs)" % (
        worst, len(units) * w.group_size, time.perf_counter() - t0))
    if worst > OUT_RTOL:
        raise SystemExit("parity check failed: %.3e > %.1e" % (worst, OUT_RTOL))
    return worst


def _oracle_unit(args):
    w, b, kv, seed = args
    os.environ["OMP_NUM_THREADS"] = "1"
    from oracle import attention, codebook, quant
    inp = _oracle_unit.inp
    ck, mk = codebook.lloyd_max(w.bits_k, w.group)
    cv, mv = codebook.lloyd_max(w.bits_v, w.group)
    so = None if inp["so4"] is None else inp["so4"][kv]
    sg = inp["signs"][kv]
    ki, kn, _ = quant.quantize(inp["k"][b, kv].astype(np.float64), sg, w.group, ck, mk, so)
    vi, vn, _ = quant.quantize(inp["v"][b, kv].astype(np.float64), sg, w.group, cv, mv, so)
    t0 = time.perf_counter()
    kd = quant.dequantize(ki, kn, sg, w.group, ck, so)
    vd = quant.dequantize(vi, vn, sg, w.group, cv, so)
    for h in range(kv * w.group_size, (kv + 1) * w.group_size):
        attention.softmax_attend(inp["q"][b, h].astype(np.float64), kd, vd, w.scale)
    return time.perf_counter() - t0


# Worker processes of the CPU baseline: the host cores this process may run on, capped at
# the CPU share of one GPU on the benchmark hosts (16 cores per GPU).
CPU_SHARE = 16


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, inp, budget_s=15.0):
    """The oracle decode on whole (sequence, KV head) streams of the same workload, one stream
    per worker process, until about budget_s of work is done.  Every codec times the same part
    in its worker: decoding the stored stream (dequantise, or decompress, or decode the keys)
    plus fp64 attention for the stream's query heads; encoding the stream is not timed.  The
    rate is the streams' token*heads over the workers' busy time divided by the workers."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits

    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, CPU_SHARE)
    _oracle_unit.inp = inp
    zip_ = w.codec in ("zip", "gtq", "qjl")
    unit_fn = {"zip": _oracle_zip_unit, "gtq": _oracle_gtq_unit, "qjl": _oracle_qjl_unit}.get(w.codec, _oracle_unit)
    units = [(w, b, kv) if zip_ else (w, b, kv, 0) for b in range(w.batch) for kv in range(w.n_kv_heads)]
    done, busy, t0 = 0, 0.0, time.perf_counter()
    with threadpool_limits(1):
        ctx = mp.get_context("fork")
        with ctx.Pool(cores) as pool:
            while done < len(units) and time.perf_counter() - t0 < budget_s:
                batch = units[done:done + cores]
                busy += sum(pool.map(unit_fn, batch))
                done += len(batch)
    wall = time.perf_counter() - t0
    token_heads = done * w.seq_len
    what = {"zip": "decompress the stored pages + fp64 attention",
            "gtq": "fp64 decode of the stored keys + attention",
            "qjl": "fp64 two-stage scores (decoded keys + residual estimate) + attention"}.get(
        w.codec, "fp64 dequantise + attention")
    return {"value": token_heads / (busy / cores), "unit": "KV token·heads/s", "cores": cores, "kind": "oracle",
            "affinity_cores": affinity, "cpu_model": cpu_model(),
            "sample": "%d of %d (sequence, KV head) streams of %s (T=%d): %s (encoding of the stream not timed), "
                      "%d worker processes x 1 thread (the host's %d available cores capped at the %d-core CPU share "
                      "of one GPU), rate over the workers' busy time %.1fs, %.1fs wall" % (
                          done, len(units), w.name, w.seq_len, what, cores, affinity, CPU_SHARE, busy, wall)}


def stream_read_probe_gbs():
    """Achievable read bandwidth: the probe kernel streaming 2 GiB (contiguous per-workgroup
    ranges, 16-byte non-temporal loads, the decode's streamed-copy policy)."""
    import ctypes

    import torch

    from compressed_domain_attention_amd import build as _b
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.tq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p]
    x = torch.ones(1 << 29, dtype=torch.float32, device="cuda")  # 2 GiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    nbytes = x.numel() * 4
    best = 0.0
    for blocks in (512, 1024, 4096):
        for _ in range(2):
            assert lib.tq_probe_stream_read(x.data_ptr(), nbytes, sink.data_ptr(), blocks, stream) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            lib.tq_probe_stream_read(x.data_ptr(), nbytes, sink.data_ptr(), blocks, stream)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 5 * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del x
    return best


COPY_BYTES = 1 << 30  # the calibration copy: bytes read and bytes written


def counter_run(w, inp, n_splits, schedule, launches=24):
    """Dispatches for a rocprofv3 --pmc pass: three copies of COPY_BYTES through the probe
    library (known traffic), then `launches` decode launches over the cache replicas, as
    bench timing issues them.  Prints nothing on stdout."""
    import ctypes

    import torch

    import compressed_domain_attention_amd as tq
    from compressed_domain_attention_amd import build as _b

    dev = torch.device("cuda:0")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.tq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.tq_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, 4096, stream) == 0
    torch.cuda.synchronize()
    del src, dst
    T = w.seq_len
    cap = (T + 31) // 32 * 32
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).to(dev)
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).to(dev), w.group, so4)
    q = torch.from_numpy(inp["q"]).to(dev)
    k0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev)
    v0 = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev)
    tq.quantize_append(rot, k0, torch.from_numpy(inp["k"]).to(dev))
    tq.quantize_append(rot, v0, torch.from_numpy(inp["v"]).to(dev))
    cache_bytes = sum(t.numel() * t.element_size() for t in (k0.codes, k0.norms, v0.codes, v0.norms))
    reps = min(256, max(2, math.ceil((1 << 30) / cache_bytes)))
    caches = [(k0, v0)] + [
        (tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev, codes=k0.codes.clone(),
                        norms=k0.norms.clone()),
         tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev, codes=v0.codes.clone(),
                        norms=v0.norms.clone())) for _ in range(reps - 1)]
    po = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    pl = torch.empty((max(n_splits, 1), w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    out = torch.empty((w.batch, w.n_q_heads, 128), dtype=torch.float32, device=dev)
    newk = torch.from_numpy(inp["k"][:, :, T - 1:T].copy()).to(dev)
    newv = torch.from_numpy(inp["v"][:, :, T - 1:T].copy()).to(dev)
    for i in range(launches):  # the launch the timed step makes
        k, v = caches[i % reps]
        if n_splits == 1:
            tq.append_decode_attention(rot, k, v, newk, newv, q, pos0=T - 1, schedule=schedule, out=out)
        else:
            tq.append_decode_attention(rot, k, v, newk, newv, q, pos0=T - 1, n_splits=n_splits, schedule=schedule,
                                       part_o=po, part_lse=pl)
    torch.cuda.synchronize()
    log("counter run: 3 copies of %d bytes, %d decode launches over %d replicas" % (COPY_BYTES, launches, reps))


def prefill_run(w, inp, launches=6):
    """Dispatches for rocprofv3 passes over the prefill: three copies of COPY_BYTES through the
    probe library (known traffic), then `launches` quantisations of the whole prompt (T - 1
    tokens of keys and values, one call each) into the same caches, as bench timing issues
    the prefill.  Prints nothing on stdout."""
    import ctypes

    import torch

    import compressed_domain_attention_amd as tq
    from compressed_domain_attention_amd import build as _b

    dev = torch.device("cuda:0")
    lib = ctypes.CDLL(_b.PROBE_LIB)
    lib.tq_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(3):
        assert lib.tq_probe_copy(src.data_ptr(), dst.data_ptr(), COPY_BYTES, 4096, stream) == 0
    torch.cuda.synchronize()
    del src, dst
    T = w.seq_len
    cap = (T + 31) // 32 * 32
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).to(dev)
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).to(dev), w.group, so4)
    k = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS, device=dev)
    v = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES, device=dev)
    pk = torch.from_numpy(inp["k"][:, :, :T - 1].copy()).to(dev)
    pv = torch.from_numpy(inp["v"][:, :, :T - 1].copy()).to(dev)
    for _ in range(launches):
        tq.quantize_append_kv(rot, k, v, pk, pv)
    torch.cuda.synchronize()
    log("prefill run: 3 copies of %d bytes, %d prefills of %d tokens" % (COPY_BYTES, launches, T - 1))


CALIBRATION_KERNEL = "(anonymous namespace)::copy_kernel("  # the probe library's copy, not torch's


def _per_dispatch(csv_path, counter, name_part):
    import csv
    import collections
    per = collections.defaultdict(float)
    for r in csv.DictReader(open(csv_path)):
        name = r["Kernel_Name"]
        hit = name.startswith(name_part) if name_part == CALIBRATION_KERNEL else name_part in name
        if r["Counter_Name"] == counter and hit:
            per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return [per[d] for d in sorted(per)]


def write_traffic(w, n_splits, fetch_csv, write_csv, commands):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) by what they read for the
    calibration copy of known size, and store HBM bytes per decode launch."""
    fc, wc = _per_dispatch(fetch_csv, "FETCH_SIZE", CALIBRATION_KERNEL), _per_dispatch(write_csv, "WRITE_SIZE", CALIBRATION_KERNEL)
    fd = _per_dispatch(fetch_csv, "FETCH_SIZE", "decode_")
    wd = _per_dispatch(write_csv, "WRITE_SIZE", "decode_")
    if not (fc and wc and fd and wd):
        raise SystemExit("counter files hold no copy or decode dispatches")
    f_factor = COPY_BYTES / (sum(fc) / len(fc) * 1024)
    w_factor = COPY_BYTES / (sum(wc) / len(wc) * 1024)
    # the first launches warm the code object; use the second half
    fd, wd = fd[len(fd) // 2:], wd[len(wd) // 2:]
    read = sum(fd) / len(fd) * 1024 * f_factor
    written = sum(wd) / len(wd) * 1024 * w_factor
    rec = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    if rec.get("kernel_sha256_16") != kernel_hash():
        rec = {"kernel_sha256_16": kernel_hash(), "workloads": {}}
    rec["workloads"]["%s/S%d" % (w.name, n_splits)] = {
        "hbm_bytes_per_launch": read + written, "read_bytes": read, "written_bytes": written,
        "algorithmic_bytes_per_launch": w.batch * w.n_kv_heads * w.seq_len * bytes_per_token_head(w),
        "fetch_scale": f_factor, "write_scale": w_factor, "commands": commands}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    log("traffic %s/S%d: read %.1f MB + written %.2f MB per launch (scales %.3f, %.3f)" % (
        w.name, n_splits, read / 1e6, written / 1e6, f_factor, w_factor))


def write_zip_traffic(w, n_splits, fetch_csv, write_csv, commands):
    """As write_traffic, for the codec's or Block-GTQ's attention kernel
    (profiles/zip_traffic.json, profiles/gtq_traffic.json)."""
    gtq = w.codec in ("gtq", "qjl")  # one kernel source, one traffic file
    kname = "gtq_attention" if gtq else "zip_attention"
    out_file = GTQ_TRAFFIC_FILE if gtq else ZIP_TRAFFIC_FILE
    khash = gtq_kernel_hash() if gtq else zip_kernel_hash()
    fc, wc = _per_dispatch(fetch_csv, "FETCH_SIZE", CALIBRATION_KERNEL), _per_dispatch(write_csv, "WRITE_SIZE", CALIBRATION_KERNEL)
    fd = _per_dispatch(fetch_csv, "FETCH_SIZE", kname)
    wd = _per_dispatch(write_csv, "WRITE_SIZE", kname)
    if not (fc and wc and fd and wd):
        raise SystemExit("counter files hold no copy or %s dispatches" % kname)
    f_factor = COPY_BYTES / (sum(fc) / len(fc) * 1024)
    w_factor = COPY_BYTES / (sum(wc) / len(wc) * 1024)
    fd, wd = fd[len(fd) // 2:], wd[len(wd) // 2:]
    read = sum(fd) / len(fd) * 1024 * f_factor
    written = sum(wd) / len(wd) * 1024 * w_factor
    rec = json.load(open(out_file)) if os.path.exists(out_file) else {}
    if rec.get("kernel_sha256_16") != khash:
        rec = {"kernel_sha256_16": khash, "workloads": {}}
    rec["workloads"]["%s/S%d" % (w.name, n_splits)] = {
        "hbm_bytes_per_launch": read + written, "read_bytes": read, "written_bytes": written,
        "fetch_scale": f_factor, "write_scale": w_factor, "commands": commands}
    os.makedirs(os.path.dirname(out_file), exist_ok=True)
    with open(out_file, "w") as f:
        json.dump(rec, f, indent=1)
    log("traffic %s/S%d: read %.1f MB + written %.2f MB per launch (scales %.3f, %.3f)" % (
        w.name, n_splits, read / 1e6, written / 1e6, f_factor, w_factor))


def schedule_sweep():
    """Decode launch time of the matrix-core and the vector schedule over the cache length T and
    the query heads per KV head (one sequence, 8 KV heads, one section, HIP-graph timing), for
    32-groups (TQ3, gqa8k's inputs) and whole-head groups with SO(4) (isoquant32k's inputs).
    Prints one table row per point."""
    from dataclasses import replace

    import torch

    import compressed_domain_attention_amd as tq

    def launch_us(fn, n=200):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (2 * n) * 1e3

    print("| group | query heads per KV head | T | matrix cores (us) | vector (us) | vector / matrix | max diff |")
    print("|---|---|---|---|---|---|---|")
    for base in ("gqa8k", "isoquant32k"):
        for g in (1, 4, 8):
            for T in (32, 64, 128, 256, 511, 512, 1024, 2048, 8192):
                w = replace(workloads.WORKLOADS[base], n_q_heads=8 * g, n_kv_heads=8).with_len(T, batch=1)
                inp = workloads.generate(w, 0)
                so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).cuda()
                rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, so4)
                cap = (T + 31) // 32 * 32
                k = tq.PackedCache(1, 8, cap, w.bits_k, w.group, tq.TQ_KEYS)
                v = tq.PackedCache(1, 8, cap, w.bits_v, w.group, tq.TQ_VALUES)
                tq.quantize_append_kv(rot, k, v, torch.from_numpy(inp["k"]).cuda(), torch.from_numpy(inp["v"]).cuda())
                q = torch.from_numpy(inp["q"]).cuda()
                out = torch.empty((1, w.n_q_heads, 128), device="cuda")
                lse = torch.empty((1, w.n_q_heads), device="cuda")
                t = {s: launch_us(lambda: tq.decode_attention(rot, k, v, q, max_len=T, schedule=s, out=out, lse=lse))
                     for s in ("mfma", "vec")}
                a, _ = tq.decode_attention(rot, k, v, q, max_len=T, schedule="mfma")
                b, _ = tq.decode_attention(rot, k, v, q, max_len=T, schedule="vec")
                torch.cuda.synchronize()
                diff = float((a - b).abs().max() / b.abs().max())
                print("| %d | %d | %d | %.2f | %.2f | %.1f | %.1e |" % (w.group, g, T, t["mfma"], t["vec"],
                                                                     t["vec"] / t["mfma"], diff), flush=True)


# the packed-cache configurations timed after the headline, in the same run and JSON line
OTHER_CONFIGS = ("long128k", "batched", "gqa8k", "tiny")


def config_summary(w, r, n_splits, probe):
    """One configuration's numbers: the decode launch against the HBM roofline (algorithmic
    bytes = codes + norms of every (token, KV head)), the whole step's rate, the sampled
    oracle check and the one-launch prefill of the prompt."""
    units = w.batch * w.n_kv_heads * w.seq_len
    algo = units * bytes_per_token_head(w)
    achieved = algo / (r["decode_ms"] / 1e3) / 1e9
    out = {
        "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "seq_len": w.seq_len,
        "bits_k": w.bits_k, "bits_v": w.bits_v, "group": w.group, "so4": w.so4, "n_splits": n_splits,
        "value": units / (r["ms_per_step"] / 1e3), "unit": "KV token·heads/s", "ms_per_step": r["ms_per_step"],
        "decode_kernel_ms": r["decode_ms"], "algorithmic_bytes_per_launch": algo,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "probe_frac": achieved / probe,
                     "traffic": measured_traffic(w.name, n_splits)},
        "prefill_ms": r["prefill_ms"], "prefill_GBps": r["prefill_bytes"] / 1e6 / r["prefill_ms"],
        "parity_worst_row_rel_err": r["parity"], "cache_replicas": r["reps"],
    }
    if r["cache_bytes"] * r["reps"] < (1 << 30):
        out["note"] = "cache-resident (%d bytes x %d replicas): a launch-latency figure" % (r["cache_bytes"], r["reps"])
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default=HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--splits", type=int, default=None)
    ap.add_argument("--schedule", default="auto", choices=["auto", "mfma", "vec"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--tail", type=int, default=0,
                    help="an unquantised tail of this many tokens per row (dense sections merged with the packed ones)")
    ap.add_argument("--tail-splits", type=int, default=None)
    ap.add_argument("--prefill-run", action="store_true",
                    help="only the prefill quantisation (after three calibration copies), for rocprofv3 passes")
    ap.add_argument("--counter-run", action="store_true",
                    help="only issue the calibration copies and decode launches (run under rocprofv3 --pmc)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) of a "
                         "--counter-run into profiles/decode_traffic.json")
    ap.add_argument("--commands", default="", help="the profiling commands, recorded with --write-traffic")
    ap.add_argument("--schedule-sweep", action="store_true",
                    help="print the decode launch time of both schedules over T and heads per KV head, then exit")
    ap.add_argument("--gtq-widths", default="1,4", metavar="LO,HI",
                    help="Block-GTQ allocation range [b_min, b_max]; above 4 bits groups take byte containers")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline configuration (the others are timed after it by default)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    global GTQ_RANGE
    GTQ_RANGE = tuple(int(x) for x in args.gtq_widths.split(","))
    if len(GTQ_RANGE) != 2 or not 1 <= GTQ_RANGE[0] <= GTQ_RANGE[1] <= 8 or GTQ_RANGE[1] - GTQ_RANGE[0] > 3:
        raise SystemExit("--gtq-widths LO,HI with 1 <= LO <= HI <= 8 and at most four widths")
    w0 = workloads.WORKLOADS[args.workload]
    if w0.codec == "gtq" and not GTQ_RANGE[0] <= w0.bits_k <= GTQ_RANGE[1]:
        raise SystemExit("--gtq-widths %d,%d cannot hold the %d-bit average budget of %s" % (
            GTQ_RANGE[0], GTQ_RANGE[1], w0.bits_k, w0.name))
    if args.schedule_sweep:
        schedule_sweep()
        return
    w = workloads.WORKLOADS[args.workload]
    n_splits = args.splits if args.splits is not None else w.n_splits
    if args.write_traffic:
        if w.codec in ("zip", "gtq", "qjl"):
            write_zip_traffic(w, n_splits, args.write_traffic[0], args.write_traffic[1], args.commands)
        else:
            write_traffic(w, n_splits, args.write_traffic[0], args.write_traffic[1], args.commands)
        return
    log("workload %s: %s, splits %d, schedule %s" % (w.name, w, n_splits, args.schedule))
    t_gen = time.perf_counter()
    inp = workloads.generate(w, 0)
    log("generated inputs in %.1fs" % (time.perf_counter() - t_gen))
    cpu = None
    if args.prefill_run:
        if w.codec != "turboquant":
            raise SystemExit("--prefill-run covers the packed-cache workloads")
        prefill_run(w, inp)
        return
    if not args.no_cpu_baseline and not args.counter_run:
        # runs before anything initialises the GPU in this process (the pool forks)
        cpu = cpu_baseline(w, inp)
        log("cpu baseline: %.3g token*heads/s (%s)" % (cpu["value"], cpu["sample"]))

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.counter_run:
        if w.codec == "zip":
            zip_counter_run(w, inp, n_splits)
        elif w.codec in ("gtq", "qjl"):
            gtq_counter_run(w, inp, n_splits)
        else:
            counter_run(w, inp, n_splits, args.schedule)
        return
    if w.codec in ("gtq", "qjl"):
        qjl = w.codec == "qjl"
        r = run_gtq(w, inp, args.steps, args.warmup, n_splits, check=not args.no_check)
        units = w.batch * w.n_kv_heads * w.seq_len
        achieved = r["algo_bytes"] / (r["attn_ms"] / 1e3) / 1e9
        probe = stream_read_probe_gbs()
        log("step %.3f ms, attention kernel %.3f ms -> %.0f GB/s (%.1f%% of 8 TB/s, %.1f%% of the %.0f GB/s probe); "
            "blocks at widths 1-8 bits: %s; %d code bytes per key; key encoding %.3f ms" % (
                r["step_ms"], r["attn_ms"], achieved, 100 * achieved / HBM_PEAK_GBS, 100 * achieved / probe, probe,
                r["widths"], r["code_bytes"], r["encode_ms"]))
        print(json.dumps({
            "metric": METRIC, "value": units / (r["step_ms"] / 1e3), "unit": "KV token·heads/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["step_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None,
            "dtype": "f16 MFMA operands (hi + lo query parts against exact +-1 codes and signs), f32 accumulate "
                     "(two-stage keys: 1-bit MSE codes + 1-bit QJL signs, 16 bytes each; fp16 values)" if qjl else
                     "f16 MFMA operands (hi + lo parts), f32 accumulate (Block-GTQ nibble%s key containers, fp16 values)"
                     % (" and byte" if r["code_bytes"] > 64 else ""),
            "data": "synthetic (seeded Gaussian activations with log-normal channel scales; workloads.py)",
            "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                       "seq_len": w.seq_len,
                       "keys": ("two-stage, %d bits: %d-bit TQ-MSE + 1-bit QJL residual" % (w.bits_k, w.bits_k - 1))
                       if qjl else "Block-GTQ, %d-bit average budget, widths %d-%d, %d code bytes per key" % (
                           w.bits_k, GTQ_RANGE[0], GTQ_RANGE[1], r["code_bytes"]),
                       "values": "fp16", "n_splits": n_splits, "timing": "HIP graph replays of up to %d consecutive steps each, over the cache replicas in turn" % STEPS_PER_GRAPH,
                       "step": "append the new token (key encoded, fp16 value) and attend over encoded keys "
                               "and fp16 values in one launch" + (", then merge" if n_splits > 1 else ""),
                       "cache_replicas": r["reps"]},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "traffic": gtq_measured_traffic(w.name, n_splits) if qjl or GTQ_RANGE == (1, 4) else None,
                         "kernel": "gtq_attention_kernel"},
            "cpu_baseline": cpu, "attention_kernel_ms": r["attn_ms"], "algorithmic_bytes_per_launch": r["algo_bytes"],
            "block_widths": r["widths"], "key_encoding_ms": r["encode_ms"], "stream_read_probe_GBps": probe,
            "parity_worst_row_rel_err": r["parity"]}), flush=True)
        return
    if w.codec == "zip":
        r = run_zip(w, inp, args.steps, args.warmup, n_splits, check=not args.no_check)
        units = w.batch * w.n_kv_heads * w.seq_len
        achieved = r["algo_bytes"] / (r["attn_ms"] / 1e3) / 1e9
        bf16_gbs = r["bf16_bytes"] / (r["attn_ms"] / 1e3) / 1e9
        probe = stream_read_probe_gbs()
        log("step %.3f ms, attention kernel %.3f ms -> %.0f GB/s of compressed pages (%.1f%% of 8 TB/s, %.1f%% of "
            "the %.0f GB/s probe); %.0f GB/s BF16-equivalent; %.1f%% of chunks kept; compress %.3f ms" % (
                r["step_ms"], r["attn_ms"], achieved, 100 * achieved / HBM_PEAK_GBS, 100 * achieved / probe, probe,
                bf16_gbs, 100 * r["kept_fraction"], r["compress_ms"]))
        print(json.dumps({
            "metric": METRIC, "value": units / (r["step_ms"] / 1e3), "unit": "KV token·heads/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["step_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16 exact (lossless codes), f32 FMA",
            "data": "synthetic (seeded Gaussian activations with outlier channels, rounded to BF16; workloads.py)",
            "config": {"workload": w.name, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                       "seq_len": w.seq_len, "codec": "lossless BF16 exponent codec (16-token pages)",
                       "n_splits": n_splits, "timing": "HIP graph replays of up to %d consecutive steps each, over the cache replicas in turn" % STEPS_PER_GRAPH,
                       "step": "attention from the compressed pages + open page" +
                               (", then merge" if n_splits > 1 else " (one section per row: no merge)"),
                       "store_replicas": r["reps"]},
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS, "traffic": zip_measured_traffic(w.name, n_splits),
                         "kernel": "zip_attention_kernel"},
            "cpu_baseline": cpu, "attention_kernel_ms": r["attn_ms"], "algorithmic_bytes_per_launch": r["algo_bytes"],
            "bf16_equivalent_GBps": bf16_gbs, "kept_chunk_fraction": r["kept_fraction"],
            "compress_ms": r["compress_ms"], "stream_read_probe_GBps": probe,
            "parity_worst_row_rel_err": r["parity"]}), flush=True)
        return
    if args.tail > w.seq_len:
        raise SystemExit("--tail takes at most the workload's %d generated tokens" % w.seq_len)
    if args.tail > 0:
        # enough sections for about 512 workgroups, at most one per 64-token chunk
        slices = -(-w.group_size // 8)
        tail_splits = args.tail_splits or max(1, min(-(-args.tail // 64), -(-512 // (w.batch * w.n_kv_heads * slices))))
        r = run_tail(w, inp, args.tail, tail_splits, args.steps, args.warmup, n_splits, args.schedule)
        units = w.batch * w.n_kv_heads * (w.seq_len + args.tail)
        dense_gbs = r["tail_bytes"] / (r["dense_ms"] / 1e3) / 1e9
        log("step %.3f ms with a %d-token %s tail; dense kernel %.4f ms -> %.0f GB/s (%.1f%% of 8 TB/s); parity %.2e" % (
            r["step_ms"], args.tail, w.dtype, r["dense_ms"], dense_gbs, 100 * dense_gbs / HBM_PEAK_GBS, r["parity"]))
        print(json.dumps({
            "metric": METRIC, "value": units / (r["step_ms"] / 1e3), "unit": "KV token·heads/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["step_ms"], "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16 MFMA operands, f32 accumulate (packed codes and fp16 tail rows; "
                     "fp32 tail rows: f32 FMA)",
            "data": "synthetic (seeded Gaussian activations with outlier channels; workloads.py)",
            "config": {"workload": "%s+tail%d" % (w.name, args.tail), "n_splits": n_splits, "tail_tokens": args.tail,
                       "tail_splits": tail_splits, "tail_dtype": w.dtype,
                       "step": "append+decode launch, dense tail launch, merge", "cache_replicas": r["reps"]},
            "roofline": {"bound": "hbm", "achieved": dense_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dense_gbs / HBM_PEAK_GBS, "traffic": None,
                         "kernel": "dense_mfma_kernel" if w.dtype == "float16" else "dense_kernel"},
            "cpu_baseline": cpu, "dense_kernel_ms": r["dense_ms"], "tail_bytes_per_launch": r["tail_bytes"],
            "parity_worst_row_rel_err": r["parity"]}), flush=True)
        return
    r = run_gpu(w, inp, args.steps, args.warmup, n_splits, args.schedule, check=not args.no_check)
    units = w.batch * w.n_kv_heads * w.seq_len
    value = units / (r["ms_per_step"] / 1e3)
    algo_bytes = units * bytes_per_token_head(w)
    achieved = algo_bytes / (r["decode_ms"] / 1e3) / 1e9
    probe = stream_read_probe_gbs()
    # every other packed-cache configuration, each with its own section count: the decode
    # launch's roofline fraction, the step rate and a sampled oracle check, in the same line
    others = {}
    if w.name == HEADLINE and not args.headline_only:
        del inp
        for name in OTHER_CONFIGS:
            torch.cuda.empty_cache()
            w2 = workloads.WORKLOADS[name]
            log("config %s: %s, splits %d" % (name, w2, w2.n_splits))
            inp2 = workloads.generate(w2, 0)
            r2 = run_gpu(w2, inp2, args.steps, args.warmup, w2.n_splits, args.schedule, check=not args.no_check)
            del inp2
            others[name] = config_summary(w2, r2, w2.n_splits, probe)
            log("  step %.4f ms, decode kernel %.4f ms -> %.0f GB/s (%.1f%% of 8 TB/s); parity %s" % (
                r2["ms_per_step"], r2["decode_ms"], others[name]["roofline"]["achieved"],
                100 * others[name]["roofline"]["frac"], r2["parity"]))
    log("step %.3f ms, decode kernel %.3f ms -> %.0f GB/s (%.1f%% of 8 TB/s, %.1f%% of the %.0f GB/s stream-read "
        "probe); prefill %.3f ms for %.2f GB (%.0f GB/s)" % (
            r["ms_per_step"], r["decode_ms"], achieved, 100 * achieved / HBM_PEAK_GBS, 100 * achieved / probe, probe,
            r["prefill_ms"], r["prefill_bytes"] / 1e9, r["prefill_bytes"] / 1e6 / r["prefill_ms"]))
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "KV token·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 MFMA operands, f32 accumulate (3/4-bit codes)",
        "data": "synthetic (seeded Gaussian activations with outlier channels; workloads.py)",
        "config": {"workload": w.name, "timing": "HIP graph replays of up to %d consecutive steps each, over the cache replicas in turn" % STEPS_PER_GRAPH, "batch": w.batch, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "seq_len": w.seq_len, "bits_k": w.bits_k, "bits_v": w.bits_v, "group": w.group,
                   "so4": w.so4, "n_splits": n_splits, "schedule": args.schedule,
                   "step": "append 1 token K+V and decode in one launch, then merge", "cache_replicas": r["reps"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": measured_traffic(w.name, n_splits)},
        "cpu_baseline": cpu,
        "decode_kernel_ms": r["decode_ms"],
        "prefill_ms": r["prefill_ms"],
        "prefill_GBps": r["prefill_bytes"] / 1e6 / r["prefill_ms"],
        "algorithmic_bytes_per_launch": algo_bytes,
        "stream_read_probe_GBps": probe,
        "parity_worst_row_rel_err": r["parity"],
    }
    if others:
        line["configs"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()

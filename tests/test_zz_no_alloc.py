"""The allocation-free decode step (section partials in the library's static device buffer)
against the step with caller-provided partial buffers followed by the merge, through the C ABI:
the same cache bytes and outputs bit for bit, on two calls in a row, the second smaller (fewer
sequences, fewer sections, shorter rows), and the capacity error for a request the static
buffer cannot hold.
"""

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


def caches(w, inp, cap, t):
    so4 = None if inp["so4"] is None else torch.from_numpy(inp["so4"]).cuda()
    rot = tq.Rotation(torch.from_numpy(inp["signs"]).cuda(), w.group, so4)
    out = []
    for _ in range(2):
        k = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_k, w.group, tq.TQ_KEYS)
        v = tq.PackedCache(w.batch, w.n_kv_heads, cap, w.bits_v, w.group, tq.TQ_VALUES)
        tq.quantize_append_kv(rot, k, v, torch.from_numpy(inp["k"][:, :, :t]).cuda(),
                              torch.from_numpy(inp["v"][:, :, :t]).cuda())
        out.append((k, v))
    return rot, out


@pytest.mark.parametrize("name", ["isoquant32k", "gqa8k", "long128k"])
def test_static_partials_equal_caller_partials(name):
    for call, (batch, seq_len, n_splits) in enumerate(((3, 300, 7), (1, 90, 3))):
        w = workloads.WORKLOADS[name].with_len(seq_len + 1, batch=batch)
        inp = workloads.generate(w, 40 + call)
        print("call %d: %s B=%d T=%d S=%d" % (call, name, batch, seq_len + 1, n_splits), flush=True)
        cap = (seq_len + 1 + 31) // 32 * 32
        rot, ((k1, v1), (k2, v2)) = caches(w, inp, cap, seq_len)
        xk = torch.from_numpy(inp["k"][:, :, seq_len:]).cuda().contiguous()
        xv = torch.from_numpy(inp["v"][:, :, seq_len:]).cuda().contiguous()
        q = torch.from_numpy(inp["q"]).cuda()
        pos = torch.tensor([seq_len - 5 * b for b in range(batch)], dtype=torch.int32, device="cuda")
        po, pl = tq.append_decode_attention(rot, k1, v1, xk, xv, q, pos=pos, n_splits=n_splits)
        ref_out, ref_lse = tq.merge_splits(rot, po, pl)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        tq.append_decode_attention_static(rot, k2, v2, xk, xv, q, out, lse, pos=pos, n_splits=n_splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        for a, b in ((k1, k2), (v1, v2)):
            assert torch.equal(a.codes, b.codes) and torch.equal(a.norms, b.norms)
        assert np.isfinite(out.cpu().numpy()).all()


def test_static_partials_capacity_and_single_section():
    w = workloads.WORKLOADS["gqa8k"].with_len(64, batch=2)
    inp = workloads.generate(w, 50)
    rot, ((k1, v1), (k2, v2)) = caches(w, inp, 64, 63)
    xk = torch.from_numpy(inp["k"][:, :, 63:]).cuda().contiguous()
    xv = torch.from_numpy(inp["v"][:, :, 63:]).cuda().contiguous()
    q = torch.from_numpy(inp["q"]).cuda()
    out = torch.zeros((w.batch, w.n_q_heads, 128), dtype=torch.float32, device="cuda")
    # 2 sequences x 32 heads x 129 floats per section: 127 sections fit in 2^20 floats, 128 do not
    before = (k2.codes.clone(), k2.norms.clone(), v2.codes.clone(), v2.norms.clone())
    with pytest.raises(tq.TQError):
        tq.append_decode_attention_static(rot, k2, v2, xk, xv, q, out, pos0=63, n_splits=128)
    torch.cuda.synchronize()
    assert not out.any()
    for a, b in zip(before, (k2.codes, k2.norms, v2.codes, v2.norms)):
        assert torch.equal(a, b)
    # one section: the step writes out itself
    ref_out, ref_lse = tq.append_decode_attention(rot, k1, v1, xk, xv, q, pos0=63, n_splits=1)
    lse = torch.empty_like(ref_lse)
    tq.append_decode_attention_static(rot, k2, v2, xk, xv, q, out, lse, pos0=63, n_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)

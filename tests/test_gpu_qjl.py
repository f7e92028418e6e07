"""GPU parity of two-stage keys (1-bit TQ-MSE + 1-bit QJL residual, oracle/qjl.py) through the
C ABI.

Every stored width of the first stage, bit-packed: one-bit codes in 16 bytes (2-bit keys),
2-bit codes in 32 bytes (3-bit keys) and 3-bit codes in 48 bytes (4-bit keys).
Encoding: MSE codes equal the oracle's except coordinates within 1e-6 of a boundary (at most
1e-5 of them, the packed cache's code bar), the MSE norm within 1e-6 relative, the residual coefficient
sqrt(pi/2)/128 |r| within 1e-4 relative (keys with a boundary code excluded: their residual
differs), and the sign bits equal the oracle's except projections within 1e-4 |r| |S_i| of
zero (the library projects the rotated-domain residual with the fp32 product S Q).
Attention is fed the oracle's records and compared with the oracle's two-stage attention
(fp64 scores <q, x_hat> + the estimate, fp16 values): within 1e-4 per row, lse within
1e-4 + 1e-5 |lse|.  Rows are ragged with an empty one; sections 1 and 3.
"""

from dataclasses import replace

import numpy as np
import pytest
import torch

import compressed_domain_attention_amd as tq
import workloads
from helpers import row_rel_err
from oracle import blockgtq as bg, qjl

pytestmark = pytest.mark.gpu

RTOL = 1e-4
LSE_ATOL = 1e-4
LSE_RTOL = 1e-5
LENS = [300, 77, 0]
BOUNDARY_EPS = 1e-6
FLIP_FRACTION = 1e-5


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    tq.library()


def case(lens=LENS, cap=320, hq=32, hkv=8, seed=0, bits_k=2):
    w = replace(workloads.WORKLOADS["qjl32k"], batch=len(lens), n_q_heads=hq, n_kv_heads=hkv, seq_len=cap,
                bits_k=bits_k)
    inp = workloads.generate(w, seed)
    bits = w.bits_k - 1  # the MSE stage
    enc = [qjl.mse_encoders(bits, inp["gauss"][h].astype(np.float64)) for h in range(hkv)]
    print("qjl case", (len(lens), hq, hkv, cap), "lens", lens, "seed", seed, "bits", bits_k, flush=True)
    return w, inp, bits, enc


def oracle_records(w, inp, enc):
    shp = (w.batch, w.n_kv_heads, w.seq_len)
    codes, norms = np.zeros(shp + (128,), np.uint8), np.zeros(shp + (4,), np.float32)
    signs, rn, xh = np.zeros(shp + (16,), np.uint8), np.zeros(shp), np.zeros(shp + (128,))
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            S = inp["proj"][h].astype(np.float64)
            c, nu, sg, r, x_hat = qjl.encode_keys(inp["k"][b, h].astype(np.float64), enc[h], S)
            codes[b, h], signs[b, h], rn[b, h], xh[b, h] = c, sg, r, x_hat
            norms[b, h, :, 0] = nu
            norms[b, h, :, 1] = np.sqrt(np.pi / 2) / 128 * r
    return codes, norms, signs, rn, xh


@pytest.mark.parametrize("bits_k", [2, 3, 4])
def test_encoding_matches_oracle(bits_k):
    w, inp, bits, enc = case(bits_k=bits_k)
    keys = tq.QjlKeys(bits, inp["gauss"], inp["proj"])
    shp = (w.batch, w.n_kv_heads, w.seq_len)
    cb = keys.code_bytes
    codes = torch.zeros(shp + (cb,), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(shp + (4,), dtype=torch.float32, device="cuda")
    signs = torch.zeros(shp + (16,), dtype=torch.uint8, device="cuda")
    x = torch.from_numpy(inp["k"]).cuda()
    tq.qjl_quantize_keys(keys, x[:, :, :100].contiguous(), codes, norms, signs, pos0=0)
    tq.qjl_quantize_keys(keys, x[:, :, 100:].contiguous(), codes, norms, signs, pos0=100)
    torch.cuda.synchronize()
    oc, on, osg, orn, oxh = oracle_records(w, inp, enc)
    got = qjl.unpack_codes(codes.cpu().numpy().reshape(-1, cb), bits).reshape(oc.shape)
    bad = got != oc
    print("first-stage code flips: %d of %d" % (bad.sum(), bad.size), flush=True)
    assert bad.mean() <= FLIP_FRACTION, bad.mean()
    for b, h, t in sorted(set(zip(*np.nonzero(bad)[:3]))):
        _, _, y = bg.quantize_keys(inp["k"][b, h, t][None].astype(np.float64), enc[h])
        for j in np.nonzero(bad[b, h, t])[0]:
            assert np.min(np.abs(enc[h][0][4] - y[0, j])) < BOUNDARY_EPS, (b, h, t, j)
    n = norms.cpu().numpy()
    assert np.allclose(n[..., 0], on[..., 0], rtol=1e-6, atol=0)
    clean = ~bad.any(axis=-1)
    assert np.allclose(n[..., 1][clean], on[..., 1][clean], rtol=1e-4, atol=0)
    assert np.all(n[..., 2:] == 0)
    # sign bits: exact except projections of the residual that are nearly zero
    gs = qjl.unpack_signs(signs.cpu().numpy())
    os_ = qjl.unpack_signs(osg)
    diff = (gs != os_) & clean[..., None]
    worst = 0
    for b, h, t in zip(*np.nonzero(diff.any(axis=-1))):
        S = inp["proj"][h].astype(np.float64)
        r = inp["k"][b, h, t].astype(np.float64) - oxh[b, h, t]
        proj = S @ r
        for i in np.nonzero(diff[b, h, t])[0]:
            assert abs(proj[i]) < 1e-4 * np.linalg.norm(r) * np.linalg.norm(S[i]), (b, h, t, i)
        worst += 1
    assert diff.mean() <= 1e-4, diff.mean()


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


@pytest.mark.parametrize("n_splits,bits_k,q_dtype", [(1, 2, np.float16), (3, 2, np.float16), (3, 3, np.float16),
                                                     (3, 2, np.float32), (1, 4, np.float16), (3, 4, np.float32)])
def test_attention_matches_oracle(n_splits, bits_k, q_dtype):
    # fp32 queries carry the same (fp16-representable) values: the oracle is unchanged
    w, inp, bits, enc = case(bits_k=bits_k)
    keys = tq.QjlKeys(bits, inp["gauss"], inp["proj"])
    oc, on, osg, orn, oxh = oracle_records(w, inp, enc)
    packed = qjl.pack_codes(oc.reshape(-1, 128), bits)
    codes = torch.from_numpy(packed.reshape(oc.shape[:3] + (keys.code_bytes,))).cuda()
    norms, signs = torch.from_numpy(on).cuda(), torch.from_numpy(osg).cuda()
    v = torch.from_numpy(inp["v"].astype(np.float16)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16).astype(q_dtype)).cuda()
    seq = torch.tensor(LENS, dtype=torch.int32, device="cuda")
    res = tq.qjl_attention(keys, codes, norms, signs, v, q, seq_lens=seq, max_len=max(LENS), scale=w.scale,
                           n_splits=n_splits)
    if n_splits > 1:
        res = tq.merge_splits(None, *res)
    torch.cuda.synchronize()
    ro = np.zeros((w.batch, w.n_q_heads, 128))
    rl = np.full((w.batch, w.n_q_heads), -np.inf)
    vf = inp["v"].astype(np.float16).astype(np.float64)
    for b, t in enumerate(LENS):
        if t == 0:
            continue
        for h in range(w.n_q_heads):
            kv = h // w.group_size
            S = inp["proj"][kv].astype(np.float64)
            qv = inp["q"][b, h].astype(np.float16).astype(np.float64)
            s = w.scale * qjl.scores(qv, oxh[b, kv, :t], osg[b, kv, :t], orn[b, kv, :t], S)
            m = s.max()
            p = np.exp(s - m)
            ro[b, h] = (p / p.sum()) @ vf[b, kv, :t]
            rl[b, h] = m + np.log(p.sum())
    check(res[0].cpu().numpy(), res[1].cpu().numpy(), ro, rl, LENS)


def device_cache(w, inp, keys):
    shp = (w.batch, w.n_kv_heads, w.seq_len)
    codes = torch.zeros(shp + (keys.code_bytes,), dtype=torch.uint8, device="cuda")
    norms = torch.zeros(shp + (4,), dtype=torch.float32, device="cuda")
    signs = torch.zeros(shp + (16,), dtype=torch.uint8, device="cuda")
    tq.qjl_quantize_keys(keys, torch.from_numpy(inp["k"]).cuda(), codes, norms, signs)
    return codes, norms, signs, torch.from_numpy(inp["v"].astype(np.float16)).cuda()


def same(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("per_row,bits_k", [(False, 2), (True, 2), (True, 3), (False, 4)])
def test_append_step_equals_encode_then_attend(per_row, bits_k):
    # one launch against encoding the new key (and writing its value) then attending: bit
    # for bit, cache and outputs; fp16 new tokens for one slot, fp32 for per-row slots
    lens = [320, 320, 320]
    w, inp, bits, enc = case(lens=lens, bits_k=bits_k)
    keys = tq.QjlKeys(bits, inp["gauss"], inp["proj"])
    rng = np.random.default_rng(9)
    dt = np.float32 if per_row else np.float16
    k_new = torch.from_numpy((rng.standard_normal((3, w.n_kv_heads, 128)) * 2).astype(dt)).cuda()
    v_new = torch.from_numpy(rng.standard_normal((3, w.n_kv_heads, 128)).astype(dt)).cuda()
    q = torch.from_numpy(inp["q"].astype(np.float16)).cuda()
    a = device_cache(w, inp, keys)
    b = tuple(t.clone() for t in a)
    if per_row:
        pos = [299, 0, 150]
        pos_d = torch.tensor(pos, dtype=torch.int32, device="cuda")
        res_a = tq.qjl_append_attention(keys, *a, k_new, v_new, q, pos=pos_d, scale=w.scale, n_splits=3)
        for r, p in enumerate(pos):
            tq.qjl_quantize_keys(keys, k_new[r:r + 1, :, None, :].contiguous(), b[0][r:r + 1], b[1][r:r + 1],
                                 b[2][r:r + 1], pos0=p)
            b[3][r, :, p] = v_new[r].half()
        res_b = tq.qjl_attention(keys, *b, q, seq_lens=pos_d + 1, max_len=max(pos) + 1, scale=w.scale, n_splits=3)
    else:
        P = 250
        res_a = tq.qjl_append_attention(keys, *a, k_new, v_new, q, pos0=P, scale=w.scale, n_splits=3)
        tq.qjl_quantize_keys(keys, k_new[:, :, None, :].contiguous(), b[0], b[1], b[2], pos0=P)
        b[3][:, :, P] = v_new
        res_b = tq.qjl_attention(keys, *b, q, max_len=P + 1, scale=w.scale, n_splits=3)
    torch.cuda.synchronize()
    assert same(a, b)
    assert same(res_a, res_b)

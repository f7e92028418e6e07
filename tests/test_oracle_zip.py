"""Pins of the lossless BF16 exponent codec oracle against the page's worked examples and
the definitions ("ZipFusion ...", compression format and register decode sections)."""

import math

import numpy as np
import pytest

from oracle import zipcodec as zc


def bf16(sign, exp, mant):
    return np.uint16((sign << 15) | (exp << 7) | mant)


def chunk_with(values, fill_exp=124, seed=0):
    """A chunk whose first entries are `values`; the rest have exponent fill_exp."""
    rng = np.random.default_rng(seed)
    x = np.array([bf16(int(rng.integers(2)), fill_exp, int(rng.integers(128))) for _ in range(zc.CHUNK)],
                 dtype=np.uint16)
    for i, v in enumerate(values):
        x[i] = v
    return x


def test_worked_example_exponent_127_with_base_120():
    # exponents 120..133 -> b = 120; exponent 127: offset 7 = 0b0111, its lowest bit stays in
    # the kept low byte and d = 3; decode: 120 + 2*3 + 1 = 127
    x = chunk_with([bf16(0, 120, 5), bf16(0, 133, 9), bf16(1, 127, 77)], fill_exp=125)
    bh, payload = zc.compress_chunk(x)
    assert bh == 60                                  # b/2
    low, codes = np.frombuffer(payload[:512], np.uint8), np.frombuffer(payload[512:], np.uint8)
    v = x[2]
    assert low[2] == (v & 0xFF) and (low[2] >> 7) == 1  # exponent's lowest bit kept
    assert codes[2] & 7 == 3                         # d = 3 (value 3 of group 0: bits 0-2)
    assert (codes[2] >> 7) == 1                      # its sign
    out = zc.decompress_chunk(bh, payload)
    assert zc.exponent(out[2]) == 127 and out[2] == v


def test_worked_example_code_byte_D0():
    # code byte 0xD0 with b/2 = 63: value 1 has sign 1, d = 0 -> high byte 128+63+0 = 0xBF;
    # value 5 has sign 1, d = 2 -> 128+63+2 = 0xC1
    x = chunk_with([bf16(1, 126, 3), 0, 0, 0, bf16(1, 130, 100)], fill_exp=127)
    x[1:4] = [bf16(0, 127, 1), bf16(0, 127, 2), bf16(0, 127, 3)]
    bh, payload = zc.compress_chunk(x)
    assert bh == 63
    codes = np.frombuffer(payload[512:], np.uint8)
    assert codes[0] == 0xD0
    out = zc.decompress_chunk(bh, payload)
    assert (out[0] >> 8) == 0xBF and (out[4] >> 8) == 0xC1
    assert out[0] == x[0] and out[4] == x[4]


def test_compress_rule_boundary():
    # b = 120 (121 rounded down to even): exponents up to 135 compress, 136 does not
    ok = chunk_with([bf16(0, 121, 0), bf16(0, 135, 0)], fill_exp=128)
    no = chunk_with([bf16(0, 121, 0), bf16(0, 136, 0)], fill_exp=128)
    assert zc.compress_chunk(ok)[0] == 60
    bh, payload = zc.compress_chunk(no)
    assert bh is None and payload == no.astype("<u2").tobytes()


@pytest.mark.parametrize("scale", [1.0, 1e-3, 300.0])
def test_round_trip_is_lossless_and_75_percent(scale):
    rng = np.random.default_rng(1)
    f = (rng.standard_normal(zc.CHUNK) * scale).astype(np.float32)
    x = (f.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any bf16 pattern will do
    bh, payload = zc.compress_chunk(x)
    assert np.array_equal(zc.decompress_chunk(bh, payload), x)
    if bh is not None:
        assert len(payload) == zc.COMPRESSED_BYTES == 3 * 2 * zc.CHUNK // 4


def test_wide_chunk_is_kept():
    rng = np.random.default_rng(2)
    x = rng.integers(0, 1 << 16, zc.CHUNK, dtype=np.uint32).astype(np.uint16)  # exponents 0..255
    bh, payload = zc.compress_chunk(x)
    assert bh is None and np.array_equal(zc.decompress_chunk(bh, payload), x)


def test_one_add_decodes_four_values():
    # the page's register trick equals the per-value rule for every code byte and base
    for b_half in range(0, 121):
        add = b_half * 0x01010101
        for c in range(256):
            word = c * 0x01010101
            first = ((word & 0x87878787) + add) & 0xFFFFFFFF
            fifth = ((((word >> 3) & 0x07070707) | ((word << 1) & 0x80808080)) + add) & 0xFFFFFFFF
            h1 = ((c >> 7) & 1) * 128 + b_half + (c & 7)
            h5 = ((c >> 6) & 1) * 128 + b_half + ((c >> 3) & 7)
            assert first == h1 * 0x01010101 and fifth == h5 * 0x01010101


@pytest.mark.parametrize("role", ["k", "v"])
def test_stream_pages_round_trip_and_metadata(role):
    rng = np.random.default_rng(3)
    t, n_pages = 70, 4                      # the tail beyond 4 full pages is not compressed
    # magnitudes in [1, 4): two exponents, so every chunk compresses
    f = (rng.uniform(1.0, 4.0, (t, 128)) * rng.choice([-1.0, 1.0], (t, 128))).astype(np.float32)
    x = (f.view(np.uint32) >> 16).astype(np.uint16)
    # makes chunk 1 of page 1 incompressible: keys' chunk 1 holds tokens 4-7 (token 20 is
    # page 1's token 4); values' chunk 1 holds coordinates 32-63
    x[20, 40] = bf16(0, 200, 0)
    store, meta = zc.compress_stream(x, n_pages, role)
    assert np.array_equal(zc.decompress_stream(store, meta, n_pages, role), x[:64])
    assert meta[1, 5] == zc.RAW
    for p in range(n_pages):
        assert int(np.frombuffer(meta[p, :4].tobytes(), "<u4")[0]) == p * zc.SLOT
        assert zc.page_bytes(meta[p]) <= zc.SLOT
    assert zc.page_bytes(meta[1]) == 3 * zc.COMPRESSED_BYTES + 2 * zc.CHUNK
    assert all(zc.page_bytes(meta[p]) == 4 * zc.COMPRESSED_BYTES for p in (0, 2, 3))


def bf16_stream(rng, t):
    # magnitudes over a few binades with random signs: most chunks compress
    f = (rng.uniform(0.25, 4.0, (t, 128)) * rng.choice([-1.0, 1.0], (t, 128))).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("role", ["k", "v"])
@pytest.mark.parametrize("t", [0, 5, 16, 70])
def test_row_tokens_reads_pages_then_open_page(t, role):
    rng = np.random.default_rng(4)
    x = bf16_stream(rng, max(t, 1))[:t]
    full = t // zc.PAGE
    store, meta = zc.compress_stream(x, max(full, 1), role) if full else (np.zeros((1, zc.SLOT), np.uint8),
                                                                           np.zeros((1, 8), np.uint8))
    # an open-page buffer of 16 rows: token i at row i mod 16; other rows are stale
    tail = bf16_stream(rng, 16)
    for i in range(full * zc.PAGE, t):
        tail[i % 16] = x[i]
    assert np.array_equal(zc.row_tokens(store, meta, tail, t, role), x)
    # a whole BF16 cache serves as the tail too (t mod rows = t)
    cache = np.concatenate([x, bf16_stream(rng, 16)])
    assert np.array_equal(zc.row_tokens(store, meta, cache, t, role), x)


def test_decode_from_pages_is_attention_on_the_original_values():
    # lossless: attention read back from pages and tail equals attention on the BF16 values
    rng = np.random.default_rng(5)
    lens = [37, 16, 0]
    bsz, hkv, g, cap = len(lens), 2, 2, 48
    x_k = np.stack([np.stack([bf16_stream(rng, cap) for _ in range(hkv)]) for _ in range(bsz)])
    x_v = np.stack([np.stack([bf16_stream(rng, cap) for _ in range(hkv)]) for _ in range(bsz)])
    q = (rng.standard_normal((bsz, hkv * g, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ks = np.zeros((bsz, hkv, 3, zc.SLOT), np.uint8)
    km = np.zeros((bsz, hkv, 3, 8), np.uint8)
    vs, vm = ks.copy(), km.copy()
    for b in range(bsz):
        for h in range(hkv):
            ks[b, h], km[b, h] = zc.compress_stream(x_k[b, h], 3, "k")
            vs[b, h], vm[b, h] = zc.compress_stream(x_v[b, h], 3, "v")
    scale = 128 ** -0.5
    out, lse = zc.decode_from_pages(q, ks, km, vs, vm, x_k, x_v, lens, scale)
    qf = zc.bf16_to_float(q)
    for b, t in enumerate(lens):
        for h in range(hkv * g):
            if t == 0:
                assert lse[b, h] == -math.inf and not out[b, h].any()
                continue
            kf, vf = zc.bf16_to_float(x_k[b, h // g, :t]), zc.bf16_to_float(x_v[b, h // g, :t])
            s = np.array([scale * sum(qf[b, h, d] * kf[j, d] for d in range(128)) for j in range(t)])
            p = np.exp(s - s.max())
            ref = (p[:, None] * vf).sum(0) / p.sum()
            assert np.allclose(out[b, h], ref, rtol=1e-12, atol=1e-12)
            assert math.isclose(lse[b, h], s.max() + math.log(p.sum()), rel_tol=1e-12)


@pytest.mark.parametrize("t,s", [(0, 3), (1, 1), (70, 1), (70, 3), (70, 8), (8200, 4), (100, 40)])
def test_sections_are_whole_pages_covering_the_row(t, s):
    b = zc.section_bounds(t, s)
    assert len(b) == s and b[0][0] == 0 and b[-1][1] == t
    for (lo, hi), (lo2, _) in zip(b, b[1:]):
        assert lo <= hi == lo2
    assert all(lo % zc.PAGE == 0 or lo == t for lo, _ in b)
    assert max(hi - lo for lo, hi in b) <= math.ceil(math.ceil(t / s) / zc.PAGE) * zc.PAGE


def test_chunk_orders_put_each_group_where_the_matrix_unit_needs_it():
    # keys: a group is 8 consecutive coordinates of one token; values: 8 consecutive tokens
    # of one coordinate; both orders are permutations of the page
    page = np.arange(zc.PAGE * zc.HEAD_DIM).reshape(zc.PAGE, zc.HEAD_DIM)
    kv = zc.page_values(page, "k").reshape(-1, 8)
    vv = zc.page_values(page, "v").reshape(-1, 8)
    t_k, d_k = np.divmod(kv, zc.HEAD_DIM)
    t_v, d_v = np.divmod(vv, zc.HEAD_DIM)
    assert (t_k == t_k[:, :1]).all() and (np.diff(d_k, axis=1) == 1).all()
    assert (d_v == d_v[:, :1]).all() and (np.diff(t_v, axis=1) == 1).all()
    # values: chunk c holds coordinates 32c .. 32c+31 of all 16 tokens
    chunks = zc.page_values(page, "v").reshape(zc.CHUNKS, -1) % zc.HEAD_DIM
    assert all(set(chunks[c]) == set(range(32 * c, 32 * c + 32)) for c in range(zc.CHUNKS))
    for role in ("k", "v"):
        assert np.array_equal(zc.page_from_values(zc.page_values(page, role), role), page)

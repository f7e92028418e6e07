"""Pins of the lossless BF16 exponent codec oracle against the page's worked examples and
the definitions ("ZipFusion ...", compression format and register decode sections)."""

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


def test_stream_pages_round_trip_and_metadata():
    rng = np.random.default_rng(3)
    t, n_pages = 70, 4                      # the tail beyond 4 full pages is not compressed
    # magnitudes in [1, 4): two exponents, so every chunk compresses
    f = (rng.uniform(1.0, 4.0, (t, 128)) * rng.choice([-1.0, 1.0], (t, 128))).astype(np.float32)
    x = (f.view(np.uint32) >> 16).astype(np.uint16)
    x[20, 5] = bf16(0, 200, 0)              # makes chunk 1 of page 1 incompressible
    store, meta = zc.compress_stream(x, n_pages)
    assert np.array_equal(zc.decompress_stream(store, meta, n_pages), x[:64])
    assert meta[1, 5] == zc.RAW
    for p in range(n_pages):
        assert int(np.frombuffer(meta[p, :4].tobytes(), "<u4")[0]) == p * zc.SLOT
        assert zc.page_bytes(meta[p]) <= zc.SLOT
    assert zc.page_bytes(meta[1]) == 3 * zc.COMPRESSED_BYTES + 2 * zc.CHUNK
    assert all(zc.page_bytes(meta[p]) == 4 * zc.COMPRESSED_BYTES for p in (0, 2, 3))

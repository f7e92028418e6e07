"""Pins for the packed layout (unit from "TurboQuant ... MNN on phones", 3.3; the layout
itself is this library's and is written out in oracle/layout.py and include/tq.h).

* hand-written worked examples (tests/golden/pack_layout_examples.txt);
* an exhaustive round trip over every 3-byte word and every 4-bit byte pair;
* an independent pure-Python bit-string writer for key records and value tiles;
* the byte counts the pages print (48 B per 128-dim 3-bit vector, ratios 4.6x / 3.6x /
  5.3x).
"""

import json
import os

import numpy as np
import pytest

from oracle import layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
FACTS = json.load(open(os.path.join(GOLDEN, "page_facts.json")))


def golden_words():
    for line in open(os.path.join(GOLDEN, "pack_layout_examples.txt")):
        if line.strip() and not line.startswith("#"):
            parts = line.split()
            bits = int(parts[1])
            codes = [int(v, 16) for v in parts[2:10]]
            data = bytes(int(v, 16) for v in parts[10:])
            yield bits, codes, data


@pytest.mark.parametrize("case", list(golden_words()))
def test_worked_examples(case):
    bits, codes, data = case
    idx = np.zeros(128, dtype=np.int64)
    idx[:8] = codes
    rec = layout.pack_keys(idx[None], bits)[0]
    assert rec[:len(data)].tobytes() == data
    assert not rec[len(data):].any()


def test_exhaustive_three_byte_words_round_trip():
    # every 24-bit pattern is exactly one set of 8 codes; run through the same bit
    # reader/writer that pack_keys / pack_values use, on bare 3-byte words
    offs8 = np.arange(8) * 3
    for chunk in np.array_split(np.arange(1 << 24, dtype=np.int64), 4):
        words = np.stack([chunk & 0xFF, (chunk >> 8) & 0xFF, (chunk >> 16) & 0xFF], axis=1).astype(np.uint8)
        offs = np.broadcast_to(offs8, (chunk.size, 8))
        codes = layout._get_bits(words, offs, 3)
        assert codes.max() <= 7
        word = np.zeros(chunk.size, dtype=np.int64)
        for j in range(8):
            word |= codes[:, j] << (3 * j)
        np.testing.assert_array_equal(word, chunk)
        back = np.zeros_like(words)
        layout._set_bits(back, offs, codes, 3)
        np.testing.assert_array_equal(back, words)
    # and the record-level wrappers on the first words of real records
    rng = np.random.default_rng(10)
    rec = rng.integers(0, 256, (4096, 48)).astype(np.uint8)
    np.testing.assert_array_equal(layout.pack_keys(layout.unpack_keys(rec, 3), 3), rec)


def test_exhaustive_nibble_bytes_round_trip():
    pairs = np.array([(a, b) for a in range(16) for b in range(16)])
    idx = np.zeros((256, 128), dtype=np.int64)
    idx[:, :2] = pairs
    rec = layout.pack_keys(idx, 4)
    np.testing.assert_array_equal(rec[:, 0], pairs[:, 0] | (pairs[:, 1] << 4))
    np.testing.assert_array_equal(layout.unpack_keys(rec, 4), idx)


def bitstring_key_record(codes, bits):
    s = "".join(format(int(c), "0%db" % bits)[::-1] for c in codes)   # LSB first per code
    return bytes(int(s[p:p + 8][::-1], 2) for p in range(0, len(s), 8))


def bitstring_value_tile(tile_codes, bits):
    """tile_codes[32][128] -> bytes, written word by word from the spec in plain Python."""
    out = bytearray()
    for q in range(4):
        for m in range(16):
            for u in range(8):
                word = 0
                for h in range(2):
                    for r in range(4):
                        t = 16 * h + 4 * q + r
                        word |= int(tile_codes[t][16 * u + m]) << (bits * (4 * h + r))
                out += word.to_bytes(bits, "little")            # 3 or 4 bytes per word
    return bytes(out)


@pytest.mark.parametrize("bits", [3, 4])
def test_independent_bitstring_writer(bits):
    rng = np.random.default_rng(11)
    idx = rng.integers(0, 2 ** bits, (64, 128))
    keys = layout.pack_keys(idx, bits)
    for t in range(0, 64, 7):
        assert keys[t].tobytes() == bitstring_key_record(idx[t], bits)
    vals = layout.pack_values(idx, bits)
    assert vals.shape == (2, 32 * 128 * bits // 8)
    for tile in range(2):
        assert vals[tile].tobytes() == bitstring_value_tile(idx[32 * tile:32 * tile + 32], bits)
    np.testing.assert_array_equal(layout.unpack_values(vals, bits), idx)
    np.testing.assert_array_equal(layout.unpack_keys(keys, bits), idx)


def test_norm_positions():
    pos = layout.norm_position(np.arange(32))
    assert sorted(pos.tolist()) == list(range(32))
    # token 16h + 4q + r sits at 8q + 4h + r: the 8 tokens of value-word group q are
    # contiguous, in slot order
    for q in range(4):
        toks = [16 * h + 4 * q + r for h in range(2) for r in range(4)]
        assert pos[toks].tolist() == list(range(8 * q, 8 * q + 8))
    rng = np.random.default_rng(12)
    n = rng.random((3, 64, 4)).astype(np.float32)
    packed = layout.pack_norms(n)
    assert packed.shape == (3, 2, 4, 32)
    assert packed[1, 1, 2, pos[5]] == n[1, 32 + 5, 2]
    np.testing.assert_array_equal(layout.unpack_norms(packed), n)


def test_byte_counts_on_pages():
    assert layout.record_bytes(3) == FACTS["isoquant_bytes_per_128dim_3bit"]["value"]
    fp16 = 128 * 2
    # 3.3: with one fp16 norm per 32-block (4 per head) the ratios are 4.6x and 3.6x
    assert round(fp16 / (layout.record_bytes(3) + 4 * 2), 1) == FACTS["tq3_compression_ratio"]["value"]
    assert round(fp16 / (layout.record_bytes(4) + 4 * 2), 1) == FACTS["tq4_compression_ratio"]["value"]
    assert (layout.record_bytes(4) + 4 * 2) * 8 / 128 == FACTS["tq4_effective_bits"]["value"]
    assert round(fp16 / layout.record_bytes(3), 1) == FACTS["isoquant_compression_codes_only"]["value"]

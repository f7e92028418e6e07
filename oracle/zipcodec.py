"""Lossless BF16 exponent codec for the KV cache (oracle).

Source: "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient LLM
Decoding" (paper-daily.com), sections on the compression format ("only the exponent is
compressed"), the page metadata and the register decode.

* A BF16 value is 1 sign bit, 8 exponent bits, 7 mantissa bits.  Within a chunk of 512
  values the exponents cluster, the mantissas do not.
* Chunk rule: b = the smallest exponent of the chunk rounded down to an even number.  If
  every exponent lies in [b, b + 15] the chunk is compressed, otherwise it is kept as is.
* Compressed value: its low byte is kept as is (7 mantissa bits and the exponent's lowest
  bit); what remains is a 4-bit code: the sign and d = (e - b) // 2 (3 bits).  8 + 4 = 12
  bits, 75% of the original.
* Decode: the high byte of a BF16 value is sign * 128 + (exponent >> 1), and
  exponent >> 1 = b/2 + d, so high = sign * 128 + b/2 + d: integer adds, no rounding.
* Code bytes: two codes per byte.  The first value's sign goes to bit 7 and its d to bits
  0-2; the fifth value's sign to bit 6 and its d to bits 3-5.  Masking a 32-bit word of 4
  code bytes with 0x87878787 gives the codes of values 1-4 in place, and a shift and mask
  those of values 5-8; one add of b/2 in every byte then yields 4 high bytes (b/2 + d is at
  most 127, so no carry crosses a byte or reaches the sign bit).
* Pages: 16 tokens.  A head's keys of one page (16 x 128 values) form 4 chunks of 512, and
  so do its values.  Per page and head, the 4 key chunks share 8 bytes of metadata (4 bytes
  for where the first chunk starts, 1 byte per chunk: "uncompressed" or b/2), and the 4
  value chunks another 8.

* Attention reads a row straight from its compressed pages: only whole pages are
  compressed; the open page (its last T mod 16 tokens) is kept uncompressed so that new
  tokens append to it ("ZipFusion ...", system overview: pages are compressed when full).

* Layout follows the matrix products: the 8 values one thread feeds the matrix unit are
  stored together, and keys and values, which play different parts in the two products
  (scores: tokens x coordinates; output: coordinates summed over tokens), are laid out
  separately ("ZipFusion ...", register decode section).

Readings (the pages leave these open): the 8 values that share 4 code bytes are 8
consecutive values of the chunk (group g = values 8g .. 8g+7, code byte 4g + j holds values
8g + j and 8g + j + 4); keys: chunk c of a page is tokens 4c .. 4c+3, token-major, so a
group is 8 consecutive coordinates of one token; values: chunk c of a page is coordinates
32c .. 32c+31 of its 16 tokens, coordinate-major (value (d - 32c) * 16 + t), so a group is
8 consecutive tokens of one coordinate; a kept chunk holds its 512 values in the same
order; a compressed chunk is its 512 low bytes, then its 256 code bytes; the
"uncompressed" mark is 0xFF (b/2 is at most 127); a page's chunks are stored back to back
from the start of a fixed 4096-byte page slot, and the 4-byte start field is the byte
offset of that slot within the (sequence, KV head) stream, little-endian; the open page's
tokens sit in a BF16 tail buffer of tail_rows rows (a multiple of 16), token t at row
t mod tail_rows; key-axis sections of a row are whole pages: C = ceil(T / S) rounded up to
a multiple of 16.
"""

import math

import numpy as np

from . import attention

PAGE = 16          # tokens per page
HEAD_DIM = 128
CHUNK = 512        # values per chunk
CHUNKS = PAGE * HEAD_DIM // CHUNK  # 4 per page per head
SLOT = CHUNKS * CHUNK * 2          # 4096 bytes: a page's chunks uncompressed
RAW = 0xFF                         # metadata mark of an uncompressed chunk
COMPRESSED_BYTES = CHUNK + CHUNK // 2  # 768


def bf16_to_float(bits):
    """BF16 bit patterns (uint16) -> float64 values: the top half of an fp32."""
    b = np.asarray(bits, dtype=np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


def exponent(bits):
    return (np.asarray(bits, dtype=np.uint32) >> 7) & 0xFF


def sign(bits):
    return np.asarray(bits, dtype=np.uint32) >> 15


def compress_chunk(bits):
    """512 BF16 bit patterns -> (b/2 or None when kept as is, payload bytes)."""
    x = np.asarray(bits, dtype=np.uint16)
    assert x.shape == (CHUNK,)
    e = exponent(x)
    b = int(e.min()) & ~1
    if int(e.max()) - b > 15:
        return None, x.astype("<u2").tobytes()
    low = (x & 0xFF).astype(np.uint8)
    d = ((e - b) >> 1).astype(np.uint32)
    s = sign(x)
    codes = np.zeros(CHUNK // 2, dtype=np.uint8)
    for g in range(CHUNK // 8):
        for j in range(4):
            i, k = 8 * g + j, 8 * g + j + 4
            codes[4 * g + j] = (s[i] << 7) | d[i] | (s[k] << 6) | (d[k] << 3)
    return b // 2, low.tobytes() + codes.tobytes()


def decompress_chunk(b_half, payload):
    """Inverse of compress_chunk, by the per-value rule high = sign*128 + b/2 + d."""
    if b_half is None:
        return np.frombuffer(payload, dtype="<u2").astype(np.uint16)
    raw = np.frombuffer(payload, dtype=np.uint8)
    low, codes = raw[:CHUNK].astype(np.uint32), raw[CHUNK:].astype(np.uint32)
    out = np.zeros(CHUNK, dtype=np.uint16)
    for g in range(CHUNK // 8):
        for j in range(4):
            c = codes[4 * g + j]
            hi1 = ((c >> 7) & 1) * 128 + b_half + (c & 7)
            hi5 = ((c >> 6) & 1) * 128 + b_half + ((c >> 3) & 7)
            out[8 * g + j] = (hi1 << 8) | low[8 * g + j]
            out[8 * g + j + 4] = (hi5 << 8) | low[8 * g + j + 4]
    return out


def page_values(page, role):
    """A page's [16][128] values in chunk order: keys token-major, values coordinate-major."""
    page = np.asarray(page)
    return (page if role == "k" else page.T).reshape(-1)


def page_from_values(vals, role):
    """Inverse of page_values: chunk-order values -> the page's [16][128] values."""
    vals = np.asarray(vals)
    return vals.reshape(PAGE, HEAD_DIM) if role == "k" else vals.reshape(HEAD_DIM, PAGE).T


def compress_stream(bits, n_pages, role):
    """One (sequence, KV head) stream of keys (role "k") or values ("v") [T >= 16 n_pages]
    [128] (uint16) -> (store bytes [n_pages][4096] uint8, metadata [n_pages][8] uint8).
    Only full pages are compressed; unused slot bytes are zero."""
    x = np.asarray(bits, dtype=np.uint16)
    store = np.zeros((n_pages, SLOT), dtype=np.uint8)
    meta = np.zeros((n_pages, 8), dtype=np.uint8)
    for p in range(n_pages):
        page = page_values(x[PAGE * p:PAGE * (p + 1)], role)
        pos = 0
        meta[p, :4] = np.frombuffer(np.uint32(p * SLOT).astype("<u4").tobytes(), dtype=np.uint8)
        for c in range(CHUNKS):
            bh, payload = compress_chunk(page[CHUNK * c:CHUNK * (c + 1)])
            store[p, pos:pos + len(payload)] = np.frombuffer(payload, dtype=np.uint8)
            pos += len(payload)
            meta[p, 4 + c] = RAW if bh is None else bh
    return store, meta


def decompress_stream(store, meta, n_pages, role):
    """Inverse of compress_stream: -> bits [16 n_pages][128] uint16."""
    out = np.zeros((n_pages * PAGE, HEAD_DIM), dtype=np.uint16)
    for p in range(n_pages):
        base = int(np.frombuffer(meta[p, :4].tobytes(), dtype="<u4")[0]) - p * SLOT  # slot-relative
        pos = base
        vals = []
        for c in range(CHUNKS):
            m = int(meta[p, 4 + c])
            n = CHUNK * 2 if m == RAW else COMPRESSED_BYTES
            vals.append(decompress_chunk(None if m == RAW else m, store[p, pos:pos + n].tobytes()))
            pos += n
        out[PAGE * p:PAGE * (p + 1)] = page_from_values(np.concatenate(vals), role)
    return out


def page_bytes(meta_row):
    """Stored bytes of one page (its 4 chunks) from its metadata row."""
    return sum(CHUNK * 2 if int(m) == RAW else COMPRESSED_BYTES for m in meta_row[4:])


def row_tokens(store, meta, tail, t, role):
    """The BF16 bits [t][128] of one (sequence, KV head) row of t tokens: pages 0 ..
    t // 16 - 1 decompressed from its store and metadata, the rest from its tail buffer
    (token i at tail row i mod len(tail), token-major for both roles)."""
    full = t // PAGE
    out = np.zeros((t, HEAD_DIM), dtype=np.uint16)
    if full:
        out[:full * PAGE] = decompress_stream(store, meta, full, role)
    for i in range(full * PAGE, t):
        out[i] = tail[i % len(tail)]
    return out


def decode_from_pages(q, k_store, k_meta, v_store, v_meta, k_tail, v_tail, seq_lens, scale):
    """Decode attention of q[B, Hq, 128] over every row's tokens read back from its
    compressed pages and tail: (out[B, Hq, 128], lse[B, Hq]) in fp64, by plain softmax
    attention on the exact BF16 values."""
    bsz, hkv = k_store.shape[:2]
    tmax = max([int(t) for t in seq_lens] + [0])
    k = np.zeros((bsz, hkv, tmax, HEAD_DIM))
    v = np.zeros((bsz, hkv, tmax, HEAD_DIM))
    for b in range(bsz):
        t = int(seq_lens[b])
        for h in range(hkv):
            k[b, h, :t] = bf16_to_float(row_tokens(k_store[b, h], k_meta[b, h], k_tail[b, h], t, "k"))
            v[b, h, :t] = bf16_to_float(row_tokens(v_store[b, h], v_meta[b, h], v_tail[b, h], t, "v"))
    return attention.decode(bf16_to_float(q), k, v, seq_lens, scale)


def section_bounds(t, n_splits):
    """Key-axis sections of a row of t tokens in whole pages: C = ceil(t / S) rounded up to
    a multiple of 16; section s is [min(t, s C), min(t, (s + 1) C))."""
    c = math.ceil(math.ceil(t / n_splits) / PAGE) * PAGE if t > 0 else 0
    return [(min(t, s * c), min(t, (s + 1) * c)) for s in range(n_splits)]

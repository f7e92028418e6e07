"""Packed byte layout of the quantised cache (oracle).

The pages fix only the packing unit: 8 three-bit indices in 3 bytes by shift and mask,
or 2 four-bit indices per byte ("TurboQuant: ... MNN on phones", 3.3), with codes and
norms kept in device memory ("RoPE-Aware Bit Allocation for KV-Cache Quantization",
packed-cache serving path).  Which 8 codes share a word, the bit order and where the
norms go are this library's layout, stated here as plainly as possible.  Head
dimension is 128 and the cache capacity is a multiple of 32 tokens (one tile).

Bit order everywhere: a word of 8 codes of b bits is the little-endian integer
sum_j code_j << (b*j), stored low byte first (3 bytes for b=3, 4 bytes for b=4).

Keys  (contraction over coordinates): one record of 128*b/8 bytes per token.  The record
      is 16 words; word w holds coordinates 8w..8w+7 of that token, slot j = 8w+j.
Values (contraction over tokens): one tile of 32 tokens is 32*128*b/8 bytes made of 512
      words.  Word W = (q*16 + m)*8 + u (q in 0..3, m in 0..15, u in 0..7) holds
      coordinate i = 16u + m of the 8 tokens t = 16h + 4q + r (h in 0..1, r in 0..3),
      token t in slot 4h + r.
Norms (keys and values alike): per tile a [groups][32] fp32 block; token t of the tile
      sits at position 8*((t >> 2) & 3) + 4*(t >> 4) + (t & 3).
"""

import numpy as np

HEAD_DIM = 128
TILE = 32


def record_bytes(bits):
    return HEAD_DIM * bits // 8


def norm_position(t):
    """Position of tile-token t (0..31) inside a tile's norm block."""
    t = np.asarray(t)
    return 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3)


def _set_bits(buf, bit_offset, value, nbits):
    """Write the low ``nbits`` of value[..., n] into buf[..., nbytes] at bit_offset[..., n].

    Bits go LSB first: bit p of the byte string is bit (p % 8) of byte p // 8.  Each bit
    position is written at most once per row, so plain assignment into an unpacked bit
    array suffices.  Leading dimensions of buf, bit_offset and value must agree.
    """
    rows_n = int(np.prod(buf.shape[:-1], dtype=np.int64))
    nbytes = buf.shape[-1]
    bitarr = np.unpackbits(buf.reshape(rows_n, nbytes), axis=-1, bitorder="little")
    offs = np.asarray(bit_offset, dtype=np.int64).reshape(rows_n, -1)
    vals = np.asarray(value, dtype=np.int64).reshape(rows_n, -1)
    for j in range(nbits):
        np.put_along_axis(bitarr, offs + j, ((vals >> j) & 1).astype(np.uint8), axis=-1)
    buf[...] = np.packbits(bitarr, axis=-1, bitorder="little").reshape(buf.shape)


def _get_bits(buf, bit_offset, nbits):
    """Read ``nbits``-bit fields at bit_offset[..., n] from buf[..., nbytes] (LSB first)."""
    rows_n = int(np.prod(buf.shape[:-1], dtype=np.int64))
    bitarr = np.unpackbits(buf.reshape(rows_n, buf.shape[-1]), axis=-1, bitorder="little")
    offs = np.asarray(bit_offset, dtype=np.int64).reshape(rows_n, -1)
    val = np.zeros(offs.shape, dtype=np.int64)
    for j in range(nbits):
        val |= np.take_along_axis(bitarr, offs + j, axis=-1).astype(np.int64) << j
    return val.reshape(bit_offset.shape)


def pack_keys(idx, bits):
    """idx[..., T, 128] -> uint8[..., T, 128*bits/8]: code i at bits [bits*i, bits*i+bits)."""
    idx = np.asarray(idx, dtype=np.int64)
    assert idx.shape[-1] == HEAD_DIM and bits in (3, 4)
    out = np.zeros(idx.shape[:-1] + (record_bytes(bits),), dtype=np.uint8)
    offs = np.broadcast_to(np.arange(HEAD_DIM) * bits, idx.shape)
    _set_bits(out, offs, idx, bits)
    return out


def unpack_keys(buf, bits):
    buf = np.asarray(buf, dtype=np.uint8)
    offs = np.broadcast_to(np.arange(HEAD_DIM) * bits, buf.shape[:-1] + (HEAD_DIM,))
    return _get_bits(buf, offs, bits).astype(np.uint8)


def _value_bit_offsets(bits):
    """[32, 128] bit offset inside a value tile of (tile-token t, coordinate i)."""
    t = np.arange(TILE)[:, None]
    i = np.arange(HEAD_DIM)[None, :]
    q = (t >> 2) & 3
    h = t >> 4
    r = t & 3
    m = i % 16
    u = i // 16
    word = (q * 16 + m) * 8 + u
    slot = 4 * h + r
    return word * (8 * bits) + bits * slot


def pack_values(idx, bits):
    """idx[..., cap, 128] (cap % 32 == 0) -> uint8[..., cap/32, 32*128*bits/8]."""
    idx = np.asarray(idx, dtype=np.int64)
    cap = idx.shape[-2]
    assert idx.shape[-1] == HEAD_DIM and cap % TILE == 0 and bits in (3, 4)
    tiles = idx.reshape(idx.shape[:-2] + (cap // TILE, TILE * HEAD_DIM))
    out = np.zeros(tiles.shape[:-1] + (TILE * record_bytes(bits),), dtype=np.uint8)
    offs = np.broadcast_to(_value_bit_offsets(bits).ravel(), tiles.shape)
    _set_bits(out, offs, tiles, bits)
    return out


def unpack_values(buf, bits):
    buf = np.asarray(buf, dtype=np.uint8)
    offs = np.broadcast_to(_value_bit_offsets(bits).ravel(), buf.shape[:-1] + (TILE * HEAD_DIM,))
    vals = _get_bits(buf, offs, bits).astype(np.uint8)
    return vals.reshape(buf.shape[:-2] + (buf.shape[-2] * TILE, HEAD_DIM))


def pack_norms(norms):
    """norms[..., cap, G] fp32 -> fp32[..., cap/32, G, 32] in tile norm order."""
    norms = np.asarray(norms, dtype=np.float32)
    cap, g = norms.shape[-2], norms.shape[-1]
    assert cap % TILE == 0
    tiles = norms.reshape(norms.shape[:-2] + (cap // TILE, TILE, g))
    out = np.zeros(norms.shape[:-2] + (cap // TILE, g, TILE), dtype=np.float32)
    pos = norm_position(np.arange(TILE))
    out[..., pos] = np.swapaxes(tiles, -1, -2)
    return out


def unpack_norms(buf):
    buf = np.asarray(buf, dtype=np.float32)
    pos = norm_position(np.arange(TILE))
    tiles = np.swapaxes(buf[..., pos], -1, -2)          # [..., cap/32, 32, G]
    return tiles.reshape(buf.shape[:-3] + (buf.shape[-3] * TILE, buf.shape[-2]))

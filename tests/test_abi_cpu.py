"""C-ABI checks that need no GPU: the library loads, exports every function include/tq.h
declares, its host-side codebook matches the oracle's, and argument errors are caught on
the host (status codes, nothing launched).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import compressed_domain_attention_amd as tq
from oracle import codebook as ocb
from oracle import qjl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")
TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_ECAPACITY = 0, 1, 2, 3
FAKE = 0x1000  # never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tq.LIB_PATH):
        pytest.fail("libtq.so is not built (run compressed_domain_attention_amd/build.py)")
    return tq.library()


def test_exports_every_declared_function(lib):
    decl = set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+(tq_\w+)\s*\(", open(HEADER).read(), re.M))
    assert decl == set(tq.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("bits,dim", [(3, 32), (4, 32), (3, 128), (4, 128)])
def test_host_codebook_matches_oracle(lib, bits, dim):
    cb = tq.make_codebook(bits, dim)
    c, m = ocb.lloyd_max(bits, dim)
    got_c = np.array(cb.centroids, dtype=np.float32)
    got_m = np.array(cb.boundaries, dtype=np.float32)
    # both round an fp64 fixed point to fp32: at most one fp32 ulp apart
    for got, ref in ((got_c, c), (got_m, m)):
        ref32 = ref.astype(np.float32)
        assert np.all(np.abs(got - ref32) <= np.spacing(np.maximum(np.abs(got), np.abs(ref32))))
    assert got_m[len(got_m) // 2] == 0.0 and m[len(m) // 2] == 0.0
    assert cb.bits == bits and cb.dim == dim
    assert all(cb.centroid[k] == 0.0 for k in range(1 << bits, 16))


@pytest.mark.parametrize("bits,dim", [(3, 32), (4, 32), (3, 128), (4, 128)])
def test_codebook_fp16_scale(lib, bits, dim):
    # the key codebook scaled by f16_scale is within the stated relative distance of fp16
    # numbers (checked with numpy's own fp16 rounding), and the scale beats no scaling
    cb = tq.make_codebook(bits, dim)
    s = np.float32(cb.f16_scale)
    assert 1.0 <= s < 2.0
    c = np.array(cb.centroids, dtype=np.float32)
    c = c[c != 0]
    def worst(scale):
        v = (np.float32(scale) * c).astype(np.float32)
        return float(np.max(np.abs(v.astype(np.float16).astype(np.float32) - v) / np.abs(v)))
    assert worst(s) <= (3e-5 if bits == 3 else 1e-4)
    assert worst(s) < worst(1.0)


def test_codebook_errors(lib):
    cb = tq.Codebook()
    assert lib.tq_make_codebook(0, 32, ctypes.byref(cb)) == TQ_EUNSUPPORTED
    assert lib.tq_make_codebook(5, 32, ctypes.byref(cb)) == TQ_EUNSUPPORTED
    assert lib.tq_make_codebook(3, 1, ctypes.byref(cb)) == TQ_EUNSUPPORTED
    assert lib.tq_make_codebook(3, 32, None) == TQ_EINVAL
    for s in range(5):
        assert lib.tq_status_string(s)
    assert lib.tq_status_string(99) == b"unknown status"


def make_rot(group=32, heads=2, so4=False):
    return tq._Rotation(group, heads, FAKE, FAKE if so4 else None)


def make_cache(role, bits=3, group=32, heads=2, batch=1, capacity=64):
    cb = tq.Codebook()
    assert tq.library().tq_make_codebook(bits, group, ctypes.byref(cb)) == 0
    return tq._Cache(FAKE, FAKE, batch, heads, capacity, bits, group, role, cb)


def append(rot, cache, n_new=4, pos=None, pos0=0, max_pos=0, x=FAKE, dtype=1):
    return tq.library().tq_quantize_append(ctypes.byref(rot), ctypes.byref(cache), x, dtype, n_new, pos, pos0,
                                           max_pos, None)


def test_append_validation(lib):
    rot = make_rot()
    k = make_cache(tq.TQ_KEYS)
    assert append(rot, k, n_new=0) == TQ_OK                      # nothing to do, nothing launched
    assert append(rot, k, n_new=65) == TQ_ECAPACITY
    assert append(rot, k, n_new=4, pos0=61) == TQ_ECAPACITY
    assert append(rot, k, n_new=4, pos=FAKE, max_pos=61) == TQ_ECAPACITY
    assert append(rot, k, x=None) == TQ_EINVAL
    assert append(rot, k, dtype=7) == TQ_EINVAL
    assert append(rot, k, n_new=-1) == TQ_EINVAL
    assert append(make_rot(group=64), k) == TQ_EUNSUPPORTED
    assert append(make_rot(heads=3), k) == TQ_EINVAL               # head count mismatch
    assert append(make_rot(group=128), k) == TQ_EINVAL             # group mismatch
    bad = make_cache(tq.TQ_KEYS, capacity=48)
    assert append(rot, bad) == TQ_EINVAL                           # capacity not a tile multiple
    bad = make_cache(tq.TQ_KEYS)
    bad.codebook.dim = 128
    assert append(rot, bad) == TQ_EINVAL                           # codebook for another group
    bad = make_cache(tq.TQ_KEYS)
    bad.bits = 2
    assert append(rot, bad) == TQ_EUNSUPPORTED
    bad = make_cache(tq.TQ_KEYS)
    bad.codebook.f16_scale = 0.0
    assert append(rot, bad) == TQ_EINVAL                           # codebook not from tq_make_codebook
    nulls = make_rot()
    nulls.signs = None
    assert append(nulls, k) == TQ_EINVAL


def append_kv(rot, k, v, n_new=4, pos=None, pos0=0, max_pos=0, xk=FAKE, xv=FAKE, dtype=1):
    return tq.library().tq_quantize_append_kv(ctypes.byref(rot), ctypes.byref(k), ctypes.byref(v), xk, xv, dtype,
                                              n_new, pos, pos0, max_pos, None)


def test_append_kv_validation(lib):
    rot = make_rot()
    k, v = make_cache(tq.TQ_KEYS), make_cache(tq.TQ_VALUES, bits=4)
    assert append_kv(rot, k, v, n_new=0) == TQ_OK
    assert append_kv(rot, k, v, n_new=65) == TQ_ECAPACITY
    assert append_kv(rot, k, v, pos=FAKE, max_pos=61) == TQ_ECAPACITY
    assert append_kv(rot, v, k) == TQ_EINVAL                       # roles swapped
    assert append_kv(rot, k, k) == TQ_EINVAL
    assert append_kv(rot, k, v, xk=None) == TQ_EINVAL
    assert append_kv(rot, k, v, xv=None) == TQ_EINVAL
    assert append_kv(rot, k, make_cache(tq.TQ_VALUES, batch=2)) == TQ_EINVAL   # batch mismatch
    assert append_kv(rot, k, make_cache(tq.TQ_VALUES, capacity=32), n_new=40) == TQ_ECAPACITY  # values only
    assert append_kv(rot, k, make_cache(tq.TQ_VALUES, group=128)) == TQ_EINVAL  # group mismatch
    assert append_kv(make_rot(heads=3), k, v) == TQ_EINVAL


def decode(rot, k, v, n_q_heads=4, max_len=10, n_splits=1, out=FAKE, part=FAKE, sched=0, scale=0.1):
    return tq.library().tq_decode_attention(ctypes.byref(rot), ctypes.byref(k), ctypes.byref(v), FAKE, 1, n_q_heads,
                                            None, max_len, scale, n_splits, sched, out, None, part, part, None)


def test_decode_validation(lib):
    rot = make_rot()
    k, v = make_cache(tq.TQ_KEYS), make_cache(tq.TQ_VALUES)
    assert decode(rot, k, k) == TQ_EINVAL                          # value cache with the key role
    assert decode(rot, k, v, n_q_heads=3) == TQ_EINVAL             # not a multiple of the KV heads
    assert decode(rot, k, v, max_len=65) == TQ_ECAPACITY
    assert decode(rot, k, v, n_splits=0) == TQ_EINVAL
    assert decode(rot, k, v, out=None) == TQ_EINVAL
    assert decode(rot, k, v, n_splits=4, part=None) == TQ_EINVAL
    assert decode(rot, k, v, sched=9) == TQ_EINVAL
    assert decode(rot, k, v, scale=float("nan")) == TQ_EINVAL
    assert decode(rot, k, make_cache(tq.TQ_VALUES, batch=2)) == TQ_EINVAL
    assert decode(rot, k, make_cache(tq.TQ_VALUES, capacity=128)) == TQ_EINVAL


def append_decode(rot, k, v, xk=FAKE, xv=FAKE, pos=None, pos0=5, max_pos=0, n_q_heads=4, n_splits=1, out=FAKE,
                  part=FAKE, sched=0, scale=0.1, q=FAKE):
    return tq.library().tq_append_decode_attention(ctypes.byref(rot), ctypes.byref(k), ctypes.byref(v), xk, xv, 1,
                                                   pos, pos0, max_pos, q, 1, n_q_heads, scale, n_splits, sched, out,
                                                   None, part, part, None)


def test_append_decode_validation(lib):
    # the one-call step rejects what either of the two calls it stands for rejects
    rot = make_rot()
    k, v = make_cache(tq.TQ_KEYS), make_cache(tq.TQ_VALUES)
    assert append_decode(rot, k, v, pos0=64) == TQ_ECAPACITY              # new token past the cache
    assert append_decode(rot, k, v, pos=FAKE, max_pos=64) == TQ_ECAPACITY
    assert append_decode(rot, k, v, pos0=-1) == TQ_EINVAL
    assert append_decode(rot, v, k) == TQ_EINVAL                          # roles swapped
    assert append_decode(rot, k, v, xk=None) == TQ_EINVAL
    assert append_decode(rot, k, v, xv=None) == TQ_EINVAL
    assert append_decode(rot, k, v, q=None) == TQ_EINVAL
    assert append_decode(rot, k, v, n_q_heads=3) == TQ_EINVAL
    assert append_decode(rot, k, v, n_splits=0) == TQ_EINVAL
    assert append_decode(rot, k, v, out=None) == TQ_EINVAL
    assert append_decode(rot, k, v, n_splits=4, part=None) == TQ_EINVAL
    assert append_decode(rot, k, v, sched=9) == TQ_EINVAL
    assert append_decode(rot, k, v, scale=float("inf")) == TQ_EINVAL
    assert append_decode(rot, k, make_cache(tq.TQ_VALUES, batch=2)) == TQ_EINVAL
    assert append_decode(rot, k, make_cache(tq.TQ_VALUES, capacity=128)) == TQ_EINVAL


def dense(rot, k=FAKE, v=FAKE, kv_dtype=1, batch=1, capacity=64, q=FAKE, n_q_heads=4, max_len=10, n_splits=1,
          part=FAKE, scale=0.1):
    return tq.library().tq_dense_attention(ctypes.byref(rot), k, v, kv_dtype, batch, capacity, q, 1, n_q_heads, None,
                                           max_len, scale, n_splits, part, part, None)


def test_dense_validation(lib):
    rot = make_rot()
    assert dense(rot, k=None) == TQ_EINVAL
    assert dense(rot, v=None) == TQ_EINVAL
    assert dense(rot, q=None) == TQ_EINVAL
    assert dense(rot, part=None) == TQ_EINVAL
    assert dense(rot, kv_dtype=7) == TQ_EINVAL
    assert dense(rot, batch=0) == TQ_EINVAL
    assert dense(rot, capacity=0) == TQ_EINVAL
    assert dense(rot, n_q_heads=3) == TQ_EINVAL
    assert dense(rot, n_splits=0) == TQ_EINVAL
    assert dense(rot, max_len=-1) == TQ_EINVAL
    assert dense(rot, max_len=65) == TQ_ECAPACITY
    assert dense(rot, scale=float("nan")) == TQ_EINVAL
    assert dense(make_rot(group=64)) == TQ_EUNSUPPORTED


def test_merge_validation(lib):
    rot = make_rot()
    m = lib.tq_merge_splits
    assert m(ctypes.byref(rot), 0, 1, 4, FAKE, FAKE, FAKE, None, None) == TQ_EINVAL
    assert m(ctypes.byref(rot), 2, 1, 3, FAKE, FAKE, FAKE, None, None) == TQ_EINVAL
    assert m(ctypes.byref(rot), 2, 1, 4, None, FAKE, FAKE, None, None) == TQ_EINVAL
    assert m(ctypes.byref(rot), 2, 1, 4, FAKE, FAKE, None, None, None) == TQ_EINVAL


def zip_compress(lib, x=FAKE, role=1, batch=1, heads=1, rows=64, src=0, dst=0, n=4, store=FAKE, meta=FAKE, pages=4):
    return lib.tq_zip_compress(x, role, batch, heads, rows, src, dst, n, store, meta, pages, None)


def test_zip_compress_validation(lib):
    assert zip_compress(lib, x=None) == TQ_EINVAL
    assert zip_compress(lib, store=None) == TQ_EINVAL
    assert zip_compress(lib, meta=None) == TQ_EINVAL
    assert zip_compress(lib, role=2) == TQ_EINVAL
    assert zip_compress(lib, batch=0) == TQ_EINVAL
    assert zip_compress(lib, heads=0) == TQ_EINVAL
    assert zip_compress(lib, rows=0) == TQ_EINVAL
    assert zip_compress(lib, pages=0) == TQ_EINVAL
    assert zip_compress(lib, src=-1) == TQ_EINVAL
    assert zip_compress(lib, dst=-1) == TQ_EINVAL
    assert zip_compress(lib, n=-1) == TQ_EINVAL
    assert zip_compress(lib, rows=63) == TQ_ECAPACITY          # page 3 needs rows 48..63
    assert zip_compress(lib, src=1) == TQ_ECAPACITY
    assert zip_compress(lib, dst=1) == TQ_ECAPACITY            # pages 1..4 of a 4-page store
    assert zip_compress(lib, pages=1 << 20) == TQ_ECAPACITY    # 32-bit start offsets
    assert zip_compress(lib, n=0) == TQ_OK                     # nothing to do, nothing launched


def zip_attn(lib, ks=FAKE, km=FAKE, vs=FAKE, vm=FAKE, pages=4, kt=FAKE, vt=FAKE, tail_rows=16, batch=1, heads=2,
             q=FAKE, q_dtype=2, hq=8, max_len=64, scale=0.1, n_splits=1, out=FAKE, part=FAKE):
    return lib.tq_zip_attention(ks, km, vs, vm, pages, kt, vt, tail_rows, batch, heads, q, q_dtype, hq, None,
                                max_len, scale, n_splits, out, None, part, part, None)


def test_zip_attention_validation(lib):
    for kw in ("ks", "km", "vs", "vm", "kt", "vt", "q"):
        assert zip_attn(lib, **{kw: None}) == TQ_EINVAL, kw
    assert zip_attn(lib, out=None) == TQ_EINVAL                 # n_splits == 1 writes out
    assert zip_attn(lib, n_splits=2, part=None) == TQ_EINVAL   # n_splits > 1 writes partials
    assert zip_attn(lib, q_dtype=3) == TQ_EINVAL
    assert zip_attn(lib, batch=0) == TQ_EINVAL
    assert zip_attn(lib, heads=0) == TQ_EINVAL
    assert zip_attn(lib, hq=7) == TQ_EINVAL                    # not a multiple of the KV heads
    assert zip_attn(lib, heads=1, hq=12) == TQ_EINVAL          # groups above 8 come in multiples of 8
    assert zip_attn(lib, tail_rows=0) == TQ_EINVAL
    assert zip_attn(lib, tail_rows=24) == TQ_EINVAL
    assert zip_attn(lib, pages=-1) == TQ_EINVAL
    assert zip_attn(lib, n_splits=0) == TQ_EINVAL
    assert zip_attn(lib, max_len=-1) == TQ_EINVAL
    assert zip_attn(lib, scale=float("inf")) == TQ_EINVAL
    assert zip_attn(lib, max_len=80) == TQ_ECAPACITY           # 4 pages + at most 15 open tokens
    assert zip_attn(lib, pages=0, max_len=17) == TQ_ECAPACITY  # no page: the tail holds every token
    assert zip_attn(lib, pages=1 << 20) == TQ_ECAPACITY


def test_merge_without_rotation_validation(lib):
    m = lib.tq_merge_splits
    assert m(None, 0, 1, 4, FAKE, FAKE, FAKE, None, None) == TQ_EINVAL
    assert m(None, 2, 0, 4, FAKE, FAKE, FAKE, None, None) == TQ_EINVAL
    assert m(None, 2, 1, 4, None, FAKE, FAKE, None, None) == TQ_EINVAL



def test_capacity_limit(lib):
    # every cache of at most TQ_MAX_CAPACITY tokens per (sequence, head) is accepted, one
    # tile more is rejected before anything is launched (32-bit offsets within a stream)
    m = re.search(r"#define TQ_MAX_CAPACITY \(1 << (\d+)\)", open(HEADER).read())
    cap = 1 << int(m.group(1))
    assert tq.MAX_CAPACITY == cap
    over = cap + tq.TILE
    rot = make_rot()
    for role in (tq.TQ_KEYS, tq.TQ_VALUES):
        assert append(rot, make_cache(role, capacity=cap), n_new=0) == TQ_OK
        assert append(rot, make_cache(role, capacity=over), n_new=0) == TQ_ECAPACITY
    k, v = make_cache(tq.TQ_KEYS, capacity=over), make_cache(tq.TQ_VALUES, capacity=over)
    assert append_kv(rot, k, v, n_new=0) == TQ_ECAPACITY
    assert decode(rot, k, v) == TQ_ECAPACITY
    assert append_decode(rot, k, v) == TQ_ECAPACITY
    assert dense(rot, capacity=over) == TQ_ECAPACITY
    qk = lib.tq_gtq_quantize_keys
    assert qk(FAKE, FAKE, FAKE, 1, 1, 1, 0, 0, cap, 64, FAKE, FAKE, None) == TQ_OK
    assert qk(FAKE, FAKE, FAKE, 1, 1, 1, 0, 0, over, 64, FAKE, FAKE, None) == TQ_ECAPACITY
    assert lib.tq_gtq_attention(FAKE, FAKE, 64, FAKE, FAKE, FAKE, over, 1, 2, FAKE, 1, 8, None, 10, 0.1, 1, FAKE, None,
                                FAKE, FAKE, None) == TQ_ECAPACITY

def test_grid_limits(lib):
    # counts that would not fit the launch grids are rejected on the host
    rot = make_rot()
    k, v = make_cache(tq.TQ_KEYS), make_cache(tq.TQ_VALUES)
    assert append(rot, make_cache(tq.TQ_KEYS, batch=32768), n_new=0) == TQ_EINVAL
    assert append(rot, make_cache(tq.TQ_KEYS, batch=32767), n_new=0) == TQ_OK
    assert decode(rot, k, v, n_splits=1 << 30) == TQ_EINVAL        # 4 heads x 2^30 sections
    assert append_decode(rot, k, v, n_splits=1 << 30) == TQ_EINVAL
    assert dense(rot, n_splits=1 << 30) == TQ_EINVAL
    assert lib.tq_merge_splits(None, 2, 1 << 16, 1 << 16, FAKE, FAKE, FAKE, None, None) == TQ_EINVAL


def test_gtq_allocate_matches_oracle(lib):
    from oracle import blockgtq as bg
    rng = np.random.default_rng(7)
    for trial in range(20):
        L = [64, 5, 17][trial % 3]
        e = np.exp(rng.standard_normal(L) * 3).astype(np.float32)
        if trial % 4 == 0:
            e[: L // 2] = e[0]  # ties
        b_min, b_max = [(1, 4), (0, 3), (2, 4)][trial % 3]
        for budget in (L * b_min, (L * (b_min + b_max)) // 2, L * b_max, L * b_min + 1):
            want = bg.allocate(e.astype(np.float64), budget, b_min, b_max)
            got = tq.gtq_allocate(e, budget, b_min, b_max)
            assert np.array_equal(want, got), (trial, budget)


def test_gtq_block_energies_match_oracle(lib):
    from oracle import blockgtq as bg
    rng = np.random.default_rng(9)
    q = (rng.standard_normal((40, 8, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    k = (rng.standard_normal((40, 2, 128)) * np.exp(rng.standard_normal(128))).astype(np.float32)
    assert np.allclose(tq.gtq_block_energies(q, k), bg.block_energies(q, k), rtol=1e-6)
    e = np.zeros(128, dtype=np.float32)
    assert lib.tq_gtq_block_energies(None, FAKE, 4, 8, 2, e.ctypes.data) == TQ_EINVAL
    assert lib.tq_gtq_block_energies(FAKE, FAKE, 4, 7, 2, e.ctypes.data) == TQ_EINVAL
    assert lib.tq_gtq_block_energies(FAKE, FAKE, 0, 8, 2, e.ctypes.data) == TQ_EINVAL


def test_gtq_allocate_validation(lib):
    e = np.ones(4, dtype=np.float32)
    b = np.zeros(4, dtype=np.int32)
    f = lib.tq_gtq_allocate
    assert f(None, 4, 8, 1, 4, b.ctypes.data) == TQ_EINVAL
    assert f(e.ctypes.data, 4, 8, 1, 4, None) == TQ_EINVAL
    assert f(e.ctypes.data, 0, 8, 1, 4, b.ctypes.data) == TQ_EINVAL
    assert f(e.ctypes.data, 4, 3, 1, 4, b.ctypes.data) == TQ_EINVAL    # below 4 x b_min
    assert f(e.ctypes.data, 4, 17, 1, 4, b.ctypes.data) == TQ_EINVAL   # above 4 x b_max
    assert f(e.ctypes.data, 4, 8, 3, 2, b.ctypes.data) == TQ_EINVAL
    bad = e.copy()
    bad[2] = -1.0
    assert f(bad.ctypes.data, 4, 8, 1, 4, b.ctypes.data) == TQ_EINVAL
    bad[2] = np.nan
    assert f(bad.ctypes.data, 4, 8, 1, 4, b.ctypes.data) == TQ_EINVAL


def test_gtq_prepare_matches_oracle(lib):
    from oracle import blockgtq as bg
    rng = np.random.default_rng(8)
    for trial in range(3):
        bits = rng.integers(1, 5, 64).astype(np.int32)
        if trial == 2:
            bits[:] = 3  # one group of all 128 coordinates
        gauss = rng.standard_normal((4, 128, 128)).astype(np.float32)
        head = tq.GtqHead()
        rot = np.zeros(tq.GTQ_ROTATION_FLOATS, dtype=np.float32)
        assert lib.tq_gtq_prepare(bits.ctypes.data, gauss.ctypes.data, ctypes.byref(head), rot.ctypes.data) == TQ_OK
        enc = bg.head_encoders(bits, gauss.astype(np.float64))
        assert head.n_groups == len(enc)
        for g, (w, coords, qm, c, m) in enumerate(enc):
            n = len(coords)
            assert head.width[g] == w and head.dim[g] == n
            assert [head.coord[head.start[g] + j] for j in range(n)] == list(coords)
            got = rot[head.rot_offset[g]:head.rot_offset[g] + n * n].reshape(n, n)
            assert np.allclose(got, qm, atol=2e-5), (trial, g)
            assert np.allclose([head.centroid[g][k] for k in range(2 ** w)], c, rtol=2e-6, atol=1e-7)
            assert np.allclose([head.boundary[g][k] for k in range(2 ** w - 1)], m, rtol=2e-6, atol=1e-7)
        assert all(head.start[g] == 128 for g in range(head.n_groups, 4))
    assert head.code_bytes == 64 and head.code_used == 64
    assert lib.tq_gtq_prepare(np.full(64, 9, np.int32).ctypes.data, gauss.ctypes.data, ctypes.byref(head),
                              rot.ctypes.data) == TQ_EINVAL
    five = np.array([1, 2, 3, 4, 5] * 12 + [1] * 4, np.int32)  # five distinct widths
    assert lib.tq_gtq_prepare(five.ctypes.data, np.zeros((5, 128, 128), np.float32).ctypes.data,
                              ctypes.byref(head), rot.ctypes.data) == TQ_EUNSUPPORTED


@pytest.mark.parametrize("widths", [(3, 5, 6), (2, 4, 7, 8), (5,), (8,)])
def test_gtq_prepare_byte_containers_match_oracle(lib, widths):
    # widths 5-8: host codebooks (Newton's method in C++) against the oracle's; the record
    # layout against the oracle's nibble/byte split
    from oracle import blockgtq as bg
    rng = np.random.default_rng(sum(widths))
    bits = np.array([widths[i % len(widths)] for i in range(64)], np.int32)
    rng.shuffle(bits)
    gauss = rng.standard_normal((8, 128, 128)).astype(np.float32)
    head = tq.GtqHead()
    rot = np.zeros(tq.GTQ_ROTATION_FLOATS, dtype=np.float32)
    assert lib.tq_gtq_prepare(bits.ctypes.data, gauss.ctypes.data, ctypes.byref(head), rot.ctypes.data) == TQ_OK
    enc = bg.head_encoders(bits, gauss.astype(np.float64))
    assert head.n_groups == len(enc)
    p = bg.nibble_positions(enc)
    assert head.code_bytes == bg.code_bytes(enc) and head.code_used == p // 2 + 128 - p
    for g, (w, coords, qm, c, m) in enumerate(enc):
        n = len(coords)
        assert head.width[g] == w and head.dim[g] == n
        assert head.byte_at[g] == (head.start[g] // 2 if w <= 4 else p // 2 + head.start[g] - p)
        cg = np.array([head.centroid[g][k] for k in range(2 ** w)])
        mg = np.array([head.boundary[g][k] for k in range(2 ** w - 1)])
        # within a few fp32 ulps of the fp64 oracle
        assert np.allclose(cg, c, rtol=4e-7, atol=2e-8), (w, n, np.max(np.abs(cg - c)))
        assert np.allclose(mg, m, rtol=4e-7, atol=2e-8), (w, n)
        assert np.all(np.diff(cg) > 0) and np.array_equal(cg, -cg[::-1])


def test_gtq_call_validation(lib):
    qk = lib.tq_gtq_quantize_keys
    assert qk(None, FAKE, FAKE, 1, 1, 1, 4, 0, 32, 64, FAKE, FAKE, None) == TQ_EINVAL
    assert qk(FAKE, FAKE, FAKE, 2, 1, 1, 4, 0, 32, 64, FAKE, FAKE, None) == TQ_EINVAL   # bf16 keys
    assert qk(FAKE, FAKE, FAKE, 1, 0, 1, 4, 0, 32, 64, FAKE, FAKE, None) == TQ_EINVAL
    for bad in (0, 48, 72, 144):  # record code bytes: 64 .. 128 in steps of 16
        assert qk(FAKE, FAKE, FAKE, 1, 1, 1, 4, 0, 32, bad, FAKE, FAKE, None) == TQ_EINVAL, bad
    assert qk(FAKE, FAKE, FAKE, 1, 1, 1, 4, 30, 32, 64, FAKE, FAKE, None) == TQ_ECAPACITY
    assert qk(FAKE, FAKE, FAKE, 1, 1, 1, 0, 0, 32, 80, FAKE, FAKE, None) == TQ_OK          # nothing launched
    at = lib.tq_gtq_attention

    def call(**kw):
        a = dict(heads=FAKE, rot=FAKE, cb=64, codes=FAKE, norms=FAKE, v=FAKE, cap=64, batch=1, hkv=2, q=FAKE, qd=1,
                 hq=8, max_len=64, scale=0.1, splits=1, out=FAKE, part=FAKE)
        a.update(kw)
        return at(a["heads"], a["rot"], a["cb"], a["codes"], a["norms"], a["v"], a["cap"], a["batch"], a["hkv"], a["q"],
                  a["qd"], a["hq"], None, a["max_len"], a["scale"], a["splits"], a["out"], None, a["part"], a["part"],
                  None)
    for k in ("heads", "rot", "codes", "norms", "v", "q"):
        assert call(**{k: None}) == TQ_EINVAL, k
    assert call(qd=2) == TQ_EINVAL
    assert call(hq=7) == TQ_EINVAL
    assert call(splits=0) == TQ_EINVAL
    assert call(out=None) == TQ_EINVAL
    assert call(splits=3, part=None) == TQ_EINVAL
    assert call(scale=float("nan")) == TQ_EINVAL
    assert call(cb=0) == TQ_EINVAL and call(cb=136) == TQ_EINVAL and call(cb=100) == TQ_EINVAL
    assert call(max_len=65) == TQ_ECAPACITY


def test_gtq_append_call_validation(lib):
    ap = lib.tq_gtq_append_attention

    def call(**kw):
        a = dict(heads=FAKE, rot=FAKE, cb=64, codes=FAKE, norms=FAKE, v=FAKE, cap=64, batch=1, hkv=2, kn=FAKE,
                 vn=FAKE, xd=1, pos=None, pos0=10, max_pos=0, q=FAKE, qd=1, hq=8, scale=0.1, splits=1, out=FAKE,
                 part=FAKE)
        a.update(kw)
        return ap(a["heads"], a["rot"], a["cb"], a["codes"], a["norms"], a["v"], a["cap"], a["batch"], a["hkv"], a["kn"],
                  a["vn"], a["xd"], a["pos"], a["pos0"], a["max_pos"], a["q"], a["qd"], a["hq"], a["scale"],
                  a["splits"], a["out"], None, a["part"], a["part"], None)
    for k in ("heads", "rot", "codes", "norms", "v", "q", "kn", "vn"):
        assert call(**{k: None}) == TQ_EINVAL, k
    assert call(xd=2) == TQ_EINVAL             # bf16 new tokens
    assert call(qd=2) == TQ_EINVAL
    assert call(pos0=-1) == TQ_EINVAL
    assert call(pos=FAKE, max_pos=-1) == TQ_EINVAL
    assert call(hq=7) == TQ_EINVAL
    assert call(splits=3, part=None) == TQ_EINVAL
    assert call(cb=32) == TQ_EINVAL
    assert call(pos0=64) == TQ_ECAPACITY       # the new slot past the capacity
    assert call(pos=FAKE, max_pos=64) == TQ_ECAPACITY


def test_qjl_projection_matches_oracle(lib):
    # proj[j][i] = (S Q)[i][j] for the one-group head the oracle's MSE stage uses
    rng = np.random.default_rng(11)
    gauss = rng.standard_normal((4, 128, 128)).astype(np.float32)
    S = rng.standard_normal((128, 128)).astype(np.float32)
    head = tq.GtqHead()
    rot = np.zeros(tq.GTQ_ROTATION_FLOATS, dtype=np.float32)
    assert lib.tq_gtq_prepare(np.full(64, 1, np.int32).ctypes.data, gauss.ctypes.data, ctypes.byref(head),
                              rot.ctypes.data) == TQ_OK
    proj = np.zeros(128 * 128, dtype=np.float32)
    assert lib.tq_gtq_qjl_projection(ctypes.byref(head), rot.ctypes.data, S.ctypes.data, proj.ctypes.data) == TQ_OK
    qm = qjl.mse_encoders(1, gauss.astype(np.float64))[0][2]
    assert np.allclose(proj.reshape(128, 128).T, S.astype(np.float64) @ qm, atol=1e-4)
    # the projection needs the one-group layout
    bits = np.full(64, 1, np.int32)
    bits[5] = 2
    assert lib.tq_gtq_prepare(bits.ctypes.data, gauss.ctypes.data, ctypes.byref(head), rot.ctypes.data) == TQ_OK
    assert lib.tq_gtq_qjl_projection(ctypes.byref(head), rot.ctypes.data, S.ctypes.data,
                                     proj.ctypes.data) == TQ_EINVAL
    assert lib.tq_gtq_qjl_projection(None, rot.ctypes.data, S.ctypes.data, proj.ctypes.data) == TQ_EINVAL


def test_qjl_call_validation(lib):
    qk = lib.tq_gtq_qjl_quantize_keys
    assert qk(FAKE, FAKE, None, 1, FAKE, 1, 1, 1, 4, 0, 32, FAKE, FAKE, FAKE, None) == TQ_EINVAL   # no projection
    assert qk(FAKE, FAKE, FAKE, 1, FAKE, 1, 1, 1, 4, 0, 32, FAKE, FAKE, None, None) == TQ_EINVAL   # no signs
    for bad in (0, 4):  # the first stage's width
        assert qk(FAKE, FAKE, FAKE, bad, FAKE, 1, 1, 1, 4, 0, 32, FAKE, FAKE, FAKE, None) == TQ_EINVAL
    assert qk(FAKE, FAKE, FAKE, 1, FAKE, 1, 1, 1, 4, 30, 32, FAKE, FAKE, FAKE, None) == TQ_ECAPACITY
    assert qk(FAKE, FAKE, FAKE, 2, FAKE, 1, 1, 1, 0, 0, 32, FAKE, FAKE, FAKE, None) == TQ_OK     # nothing launched
    at = lib.tq_gtq_qjl_attention

    def call(**kw):
        a = dict(proj=FAKE, bits=1, signs=FAKE, codes=FAKE, max_len=64, splits=1, out=FAKE)
        a.update(kw)
        return at(FAKE, FAKE, a["proj"], a["bits"], a["codes"], FAKE, a["signs"], FAKE, 64, 1, 2, FAKE, 1, 8, None,
                  a["max_len"], 0.1, a["splits"], a["out"], None, FAKE, FAKE, None)
    assert call(proj=None) == TQ_EINVAL and call(signs=None) == TQ_EINVAL and call(codes=None) == TQ_EINVAL
    assert call(out=None) == TQ_EINVAL and call(max_len=65) == TQ_ECAPACITY
    assert call(bits=0) == TQ_EINVAL and call(bits=4) == TQ_EINVAL


def test_product_path_has_no_cpu_fallback():
    # the binding must not reach the oracle or any CPU computation
    src = open(os.path.join(ROOT, "compressed_domain_attention_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("NativeLibraryMissing", "")


def test_binding_rejects_host_tensors_and_wrong_buffers(lib):
    # the binding hands raw addresses to the kernels: host tensors and caller buffers that do
    # not match the cache layout are refused before any call
    import torch
    with pytest.raises(ValueError, match="current GPU"):
        tq.PackedCache(1, 2, 64, 3, 32, tq.TQ_KEYS, device="cpu")
    with pytest.raises(ValueError, match="current GPU"):
        tq.Rotation(torch.ones(2, 128), 32)
    with pytest.raises(ValueError, match="signs must be"):
        tq.Rotation(torch.ones(2, 64), 32)
    with pytest.raises(ValueError, match="so4 must be"):
        tq.Rotation(torch.ones(2, 128), 128, torch.zeros(2, 16, 2, 4))
    with pytest.raises(ValueError, match="codes must be"):
        tq.PackedCache(1, 2, 64, 3, 32, tq.TQ_KEYS, codes=torch.zeros(1, 2, 32, 48, dtype=torch.uint8),
                       norms=torch.zeros(1, 2, 2, 4, 32))
    with pytest.raises(ValueError, match="norms must be"):
        tq.PackedCache(1, 2, 64, 3, 32, tq.TQ_KEYS, codes=torch.zeros(1, 2, 64, 48, dtype=torch.uint8),
                       norms=torch.zeros(1, 2, 2, 4, 32, dtype=torch.float64))

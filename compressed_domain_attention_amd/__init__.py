"""Compressed-domain decode attention on a packed 3/4-bit KV cache, for MI355X (gfx950).

Thin ctypes binding over ``libtq.so`` (C ABI in ``include/tq.h``).  This module only
marshals arguments: it allocates cache buffers with PyTorch (device memory is PyTorch's
job here), fills the C structs, and passes raw device pointers plus the current HIP
stream.  Every step of quantisation and attention runs in the library's HIP kernels.
There is no fallback: if the library is missing the calls raise ``NativeLibraryMissing``.
"""

import ctypes
import math
import os

import torch

__all__ = [
    "NativeLibraryMissing", "TQError", "Codebook", "make_codebook", "Rotation", "PackedCache",
    "quantize_append", "decode_attention", "merge_splits", "library", "LIB_PATH",
    "zip_store", "zip_compress", "zip_attention",
    "gtq_block_energies", "gtq_allocate", "GtqKeys", "gtq_quantize_keys", "gtq_attention", "gtq_append_attention",
    "QjlKeys", "qjl_quantize_keys", "qjl_attention", "qjl_append_attention",
    "TQ_KEYS", "TQ_VALUES",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")
HEAD_DIM = 128
TILE = 32
MAX_CAPACITY = 1 << 24  # tokens per (sequence, head) of any cache
TQ_KEYS = 0
TQ_VALUES = 1
_SCHEDULES = {"auto": 0, "vec": 1, "mfma": 2}
_DTYPES = {torch.float32: 0, torch.float16: 1}
_ZIP_Q_DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
ZIP_PAGE = 16      # tokens per compressed page
ZIP_SLOT = 4096    # bytes of one page's slot in the store


class NativeLibraryMissing(RuntimeError):
    pass


class TQError(RuntimeError):
    def __init__(self, status, what):
        super().__init__("%s: %s (status %d)" % (what, _status_string(status), status))
        self.status = status


class Codebook(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("dim", ctypes.c_int32),
                ("centroid", ctypes.c_float * 16), ("boundary", ctypes.c_float * 15), ("f16_scale", ctypes.c_float)]

    @property
    def centroids(self):
        return [self.centroid[k] for k in range(1 << self.bits)]

    @property
    def boundaries(self):
        return [self.boundary[k] for k in range((1 << self.bits) - 1)]


class _Rotation(ctypes.Structure):
    _fields_ = [("group", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("signs", ctypes.c_void_p), ("so4", ctypes.c_void_p)]


class GtqHead(ctypes.Structure):
    """tq_gtq_head: one KV head's Block-GTQ key encoder (layout in include/tq.h)."""
    _fields_ = [("n_groups", ctypes.c_int32), ("width", ctypes.c_int32 * 4), ("start", ctypes.c_int32 * 4),
                ("dim", ctypes.c_int32 * 4), ("rot_offset", ctypes.c_int32 * 4), ("coord", ctypes.c_int32 * 128),
                ("byte_at", ctypes.c_int32 * 4), ("code_used", ctypes.c_int32), ("code_bytes", ctypes.c_int32),
                ("centroid", (ctypes.c_float * 256) * 4), ("boundary", (ctypes.c_float * 255) * 4),
                ("f16_scale", ctypes.c_float * 4)]


class _Cache(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("norms", ctypes.c_void_p), ("batch", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("capacity", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("role", ctypes.c_int32), ("codebook", Codebook)]


_lib = None

EXPORTS = ("tq_status_string", "tq_make_codebook", "tq_quantize_append", "tq_quantize_append_kv",
           "tq_decode_attention", "tq_append_decode_attention", "tq_append_decode_attention_static",
           "tq_dense_attention", "tq_merge_splits",
           "tq_zip_compress", "tq_zip_attention", "tq_gtq_block_energies", "tq_gtq_allocate", "tq_gtq_prepare", "tq_gtq_quantize_keys",
           "tq_gtq_attention", "tq_gtq_append_attention", "tq_gtq_qjl_projection", "tq_gtq_qjl_quantize_keys",
           "tq_gtq_qjl_attention", "tq_gtq_qjl_append_attention")


def library():
    """Load libtq.so once; raise NativeLibraryMissing if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NativeLibraryMissing("%s is not built: run `python compressed_domain_attention_amd/build.py`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.tq_status_string.argtypes = [I]
    lib.tq_status_string.restype = ctypes.c_char_p
    lib.tq_make_codebook.argtypes = [I, I, ctypes.POINTER(Codebook)]
    lib.tq_make_codebook.restype = I
    lib.tq_quantize_append.argtypes = [ctypes.POINTER(_Rotation), ctypes.POINTER(_Cache), P, I, I, P, I, I, P]
    lib.tq_quantize_append.restype = I
    lib.tq_quantize_append_kv.argtypes = [ctypes.POINTER(_Rotation), ctypes.POINTER(_Cache), ctypes.POINTER(_Cache),
                                          P, P, I, I, P, I, I, P]
    lib.tq_quantize_append_kv.restype = I
    lib.tq_decode_attention.argtypes = [ctypes.POINTER(_Rotation), ctypes.POINTER(_Cache), ctypes.POINTER(_Cache),
                                        P, I, I, P, I, F, I, I, P, P, P, P, P]
    lib.tq_decode_attention.restype = I
    lib.tq_append_decode_attention.argtypes = [ctypes.POINTER(_Rotation), ctypes.POINTER(_Cache),
                                               ctypes.POINTER(_Cache), P, P, I, P, I, I, P, I, I, F, I, I, P, P, P,
                                               P, P]
    lib.tq_append_decode_attention.restype = I
    lib.tq_append_decode_attention_static.argtypes = [ctypes.POINTER(_Rotation), ctypes.POINTER(_Cache),
                                                      ctypes.POINTER(_Cache), P, P, I, P, I, I, P, I, I, F, I, I,
                                                      P, P, P]
    lib.tq_append_decode_attention_static.restype = I
    lib.tq_dense_attention.argtypes = [ctypes.POINTER(_Rotation), P, P, I, I, I, P, I, I, P, I, F, I, P, P, P]
    lib.tq_dense_attention.restype = I
    lib.tq_merge_splits.argtypes = [ctypes.POINTER(_Rotation), I, I, I, P, P, P, P, P]
    lib.tq_merge_splits.restype = I
    lib.tq_zip_compress.argtypes = [P, I, I, I, I, I, I, I, P, P, I, P]
    lib.tq_zip_compress.restype = I
    lib.tq_zip_attention.argtypes = [P, P, P, P, I, P, P, I, I, I, P, I, I, P, I, F, I, P, P, P, P, P]
    lib.tq_zip_attention.restype = I
    lib.tq_gtq_block_energies.argtypes = [P, P, I, I, I, P]
    lib.tq_gtq_block_energies.restype = I
    lib.tq_gtq_allocate.argtypes = [P, I, I, I, I, P]
    lib.tq_gtq_allocate.restype = I
    lib.tq_gtq_prepare.argtypes = [P, P, ctypes.POINTER(GtqHead), P]
    lib.tq_gtq_prepare.restype = I
    lib.tq_gtq_quantize_keys.argtypes = [P, P, P, I, I, I, I, I, I, I, P, P, P]
    lib.tq_gtq_quantize_keys.restype = I
    lib.tq_gtq_attention.argtypes = [P, P, I, P, P, P, I, I, I, P, I, I, P, I, F, I, P, P, P, P, P]
    lib.tq_gtq_attention.restype = I
    lib.tq_gtq_append_attention.argtypes = [P, P, I, P, P, P, I, I, I, P, P, I, P, I, I, P, I, I, F, I, P, P, P, P,
                                            P]
    lib.tq_gtq_append_attention.restype = I
    lib.tq_gtq_qjl_projection.argtypes = [P, P, P, P]
    lib.tq_gtq_qjl_projection.restype = I
    lib.tq_gtq_qjl_quantize_keys.argtypes = [P, P, P, I, P, I, I, I, I, I, I, P, P, P, P]
    lib.tq_gtq_qjl_quantize_keys.restype = I
    lib.tq_gtq_qjl_attention.argtypes = [P, P, P, I, P, P, P, P, I, I, I, P, I, I, P, I, F, I, P, P, P, P, P]
    lib.tq_gtq_qjl_attention.restype = I
    lib.tq_gtq_qjl_append_attention.argtypes = [P, P, P, I, P, P, P, P, I, I, I, P, P, I, P, I, I, P, I, I, F, I, P,
                                                P, P, P, P]
    lib.tq_gtq_qjl_append_attention.restype = I
    _lib = lib
    return lib


def _status_string(status):
    try:
        return library().tq_status_string(status).decode()
    except NativeLibraryMissing:
        return "unknown"


def _check(status, what):
    if status != 0:
        raise TQError(status, what)


def _device_ptr(t, what="tensor"):
    """The raw address of a tensor the kernels read or write: it must live on the current GPU
    (a host address passed to a kernel would fault the device)."""
    if not t.is_cuda or t.device.index != torch.cuda.current_device():
        raise ValueError("%s must be on the current GPU (cuda:%d), not %s" % (
            what, torch.cuda.current_device() if torch.cuda.is_available() else 0, t.device))
    return t.data_ptr()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(_device_ptr(t))


def _need(t, shape, dtypes, name):
    """Refuse a tensor that the call would address in another size, type or layout."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype not in dtypes or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %s tensor of shape %s, not %s %s" % (
            name, "/".join(str(d).replace("torch.", "") for d in dtypes), tuple(shape),
            str(t.dtype).replace("torch.", ""), tuple(t.shape)))


def _outputs(n_splits, bsz, hq, dev, out, lse, part_o, part_lse):
    """The attention calls' outputs: caller buffers checked, missing ones allocated."""
    f32 = (torch.float32,)
    if n_splits == 1:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=dev) if out is None else out
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=dev) if lse is None else lse
        _need(out, (bsz, hq, HEAD_DIM), f32, "out")
        _need(lse, (bsz, hq), f32, "lse")
    else:
        if part_o is None:
            part_o = torch.empty((n_splits, bsz, hq, HEAD_DIM), dtype=torch.float32, device=dev)
        if part_lse is None:
            part_lse = torch.empty((n_splits, bsz, hq), dtype=torch.float32, device=dev)
        _need(part_o, (n_splits, bsz, hq, HEAD_DIM), f32, "part_o")
        _need(part_lse, (n_splits, bsz, hq), f32, "part_lse")
    return out, lse, part_o, part_lse


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_codebook(bits: int, dim: int) -> Codebook:
    """Lloyd-Max codebook for dimension ``dim`` (host computation inside the library)."""
    cb = Codebook()
    _check(library().tq_make_codebook(bits, dim, ctypes.byref(cb)), "tq_make_codebook")
    return cb


class Rotation:
    """Per-KV-head rotation: signs [H, 128] (+-1) and optional SO(4) pairs [H, 32, 2, 4]."""

    def __init__(self, signs: torch.Tensor, group: int, so4: torch.Tensor = None):
        self.signs = signs.contiguous().to(torch.float32)
        self.so4 = None if so4 is None else so4.contiguous().to(torch.float32)
        self.group = group
        self.n_kv_heads = self.signs.shape[0]
        if self.signs.dim() != 2 or self.signs.shape[1] != HEAD_DIM:
            raise ValueError("signs must be [n_kv_heads, %d]" % HEAD_DIM)
        if self.so4 is not None and tuple(self.so4.shape) != (self.n_kv_heads, HEAD_DIM // 4, 2, 4):
            raise ValueError("so4 must be [n_kv_heads, %d, 2, 4]" % (HEAD_DIM // 4))
        self.c = _Rotation(group, self.n_kv_heads, _device_ptr(self.signs, "signs"),
                           None if self.so4 is None else _device_ptr(self.so4, "so4"))


class PackedCache:
    """Caller-owned packed keys or values: codes + fp32 group norms, layout of include/tq.h."""

    def __init__(self, batch, n_kv_heads, capacity, bits, group, role, device="cuda", codebook=None,
                 codes=None, norms=None):
        if capacity % TILE:
            raise ValueError("capacity must be a multiple of %d" % TILE)
        self.batch, self.n_kv_heads, self.capacity = batch, n_kv_heads, capacity
        self.bits, self.group, self.role = bits, group, role
        self.codebook = codebook if codebook is not None else make_codebook(bits, group)
        ng = HEAD_DIM // group
        shape = ((batch, n_kv_heads, capacity, 16 * bits) if role == TQ_KEYS
                 else (batch, n_kv_heads, capacity // TILE, TILE * 16 * bits))
        nshape = (batch, n_kv_heads, capacity // TILE, ng, TILE)
        if codes is None:
            codes = torch.zeros(shape, dtype=torch.uint8, device=device)
        if norms is None:
            norms = torch.zeros(nshape, dtype=torch.float32, device=device)
        # caller-supplied buffers: the kernels address them by the layout, so it must match
        if codes.dtype != torch.uint8 or codes.numel() != math.prod(shape) or not codes.is_contiguous():
            raise ValueError("codes must be a contiguous uint8 tensor of %s elements" % (shape,))
        if norms.dtype != torch.float32 or norms.numel() != math.prod(nshape) or not norms.is_contiguous():
            raise ValueError("norms must be a contiguous float32 tensor of %s elements" % (nshape,))
        self.codes, self.norms = codes, norms
        self.c = _Cache(_device_ptr(codes, "codes"), _device_ptr(norms, "norms"), batch, n_kv_heads, capacity, bits,
                        group, role, self.codebook)


def quantize_append(rot: Rotation, cache: PackedCache, x: torch.Tensor, pos: torch.Tensor = None, pos0: int = 0,
                    max_pos: int = None):
    """Quantise x [batch, n_kv_heads, n_new, 128] (fp16/fp32) into slots pos.. of the cache."""
    if x.dtype not in _DTYPES or not x.is_contiguous():
        raise ValueError("x must be a contiguous float16/float32 tensor")
    n_new = x.shape[2] if x.dim() == 4 else -1
    _need(x, (cache.batch, cache.n_kv_heads, n_new, HEAD_DIM), tuple(_DTYPES), "x")
    _need(pos, (cache.batch,), (torch.int32,), "pos")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    _check(library().tq_quantize_append(ctypes.byref(rot.c), ctypes.byref(cache.c), _ptr(x), _DTYPES[x.dtype],
                                        n_new, _ptr(pos), pos0, max_pos, _stream()), "tq_quantize_append")


def quantize_append_kv(rot: Rotation, keys: PackedCache, values: PackedCache, xk: torch.Tensor, xv: torch.Tensor,
                       pos: torch.Tensor = None, pos0: int = 0, max_pos: int = None):
    """Quantise new keys xk and values xv [batch, n_kv_heads, n_new, 128] in one launch."""
    for x in (xk, xv):
        if x.dtype not in _DTYPES or not x.is_contiguous():
            raise ValueError("xk and xv must be contiguous float16/float32 tensors")
    if xk.dtype != xv.dtype or xk.shape != xv.shape:
        raise ValueError("xk and xv must have the same dtype and shape")
    n_new = xk.shape[2] if xk.dim() == 4 else -1
    _need(xk, (keys.batch, keys.n_kv_heads, n_new, HEAD_DIM), tuple(_DTYPES), "xk")
    _need(pos, (keys.batch,), (torch.int32,), "pos")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    _check(library().tq_quantize_append_kv(ctypes.byref(rot.c), ctypes.byref(keys.c), ctypes.byref(values.c),
                                           _ptr(xk), _ptr(xv), _DTYPES[xk.dtype], xk.shape[2], _ptr(pos), pos0,
                                           max_pos, _stream()), "tq_quantize_append_kv")


def decode_attention(rot: Rotation, keys: PackedCache, values: PackedCache, q: torch.Tensor, seq_lens=None,
                     max_len=None, scale=None, n_splits=1, schedule="auto", out=None, lse=None, part_o=None,
                     part_lse=None):
    """One decode step.  n_splits == 1 -> (out, lse); n_splits > 1 -> (part_o, part_lse)."""
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    bsz, hq = keys.batch, q.shape[1] if q.dim() == 3 else -1
    _need(q, (bsz, hq, HEAD_DIM), tuple(_DTYPES), "q")
    _need(seq_lens, (bsz,), (torch.int32,), "seq_lens")
    if max_len is None:
        max_len = int(seq_lens.max().item()) if seq_lens is not None else keys.capacity
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_decode_attention(
        ctypes.byref(rot.c), ctypes.byref(keys.c), ctypes.byref(values.c), _ptr(q), _DTYPES[q.dtype], hq,
        _ptr(seq_lens), max_len, scale, n_splits, _SCHEDULES[schedule], _ptr(out), _ptr(lse), _ptr(part_o),
        _ptr(part_lse), _stream()), "tq_decode_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


def append_decode_attention(rot: Rotation, keys: PackedCache, values: PackedCache, xk: torch.Tensor,
                            xv: torch.Tensor, q: torch.Tensor, pos: torch.Tensor = None, pos0: int = 0,
                            max_pos: int = None, scale=None, n_splits=1, schedule="auto", out=None, lse=None,
                            part_o=None, part_lse=None):
    """Append one new key/value token per (sequence, KV head) at pos (or pos0), then decode
    over rows ending at it, in one call.  Returns as decode_attention."""
    for x in (xk, xv):
        if x.dtype not in _DTYPES or not x.is_contiguous():
            raise ValueError("xk and xv must be contiguous float16/float32 tensors")
    if xk.dtype != xv.dtype or xk.shape != xv.shape or xk.shape[2] != 1:
        raise ValueError("xk and xv must have the same dtype and shape, one token per stream")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    _need(xk, (keys.batch, keys.n_kv_heads, 1, HEAD_DIM), tuple(_DTYPES), "xk")
    _need(q, (keys.batch, q.shape[1] if q.dim() == 3 else -1, HEAD_DIM), tuple(_DTYPES), "q")
    _need(pos, (keys.batch,), (torch.int32,), "pos")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_append_decode_attention(
        ctypes.byref(rot.c), ctypes.byref(keys.c), ctypes.byref(values.c), _ptr(xk), _ptr(xv), _DTYPES[xk.dtype],
        _ptr(pos), pos0, max_pos, _ptr(q), _DTYPES[q.dtype], hq, scale, n_splits, _SCHEDULES[schedule], _ptr(out),
        _ptr(lse), _ptr(part_o), _ptr(part_lse), _stream()), "tq_append_decode_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


STATIC_PARTIAL_FLOATS = 1 << 20  # the library's static partial buffer, floats per device


def append_decode_attention_static(rot: Rotation, keys: PackedCache, values: PackedCache, xk: torch.Tensor,
                                   xv: torch.Tensor, q: torch.Tensor, out: torch.Tensor, lse: torch.Tensor = None,
                                   pos: torch.Tensor = None, pos0: int = 0, max_pos: int = None, scale=None,
                                   n_splits=1, schedule="auto"):
    """append_decode_attention with n_splits sections and the merge, the section partials in
    the library's static device buffer (no allocation by the call): writes out [batch, n_q_heads,
    128] fp32 and, if given, lse [batch, n_q_heads]; returns (out, lse)."""
    for x in (xk, xv):
        if x.dtype not in _DTYPES or not x.is_contiguous():
            raise ValueError("xk and xv must be contiguous float16/float32 tensors")
    if xk.dtype != xv.dtype or xk.shape != xv.shape or xk.shape[2] != 1:
        raise ValueError("xk and xv must have the same dtype and shape, one token per stream")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    _need(xk, (keys.batch, keys.n_kv_heads, 1, HEAD_DIM), tuple(_DTYPES), "xk")
    _need(q, (keys.batch, q.shape[1] if q.dim() == 3 else -1, HEAD_DIM), tuple(_DTYPES), "q")
    _need(pos, (keys.batch,), (torch.int32,), "pos")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    if tuple(out.shape) != (bsz, hq, HEAD_DIM) or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [batch, n_q_heads, 128]")
    if lse is not None and (tuple(lse.shape) != (bsz, hq) or lse.dtype != torch.float32 or not lse.is_contiguous()):
        raise ValueError("lse must be contiguous float32 [batch, n_q_heads]")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    _check(library().tq_append_decode_attention_static(
        ctypes.byref(rot.c), ctypes.byref(keys.c), ctypes.byref(values.c), _ptr(xk), _ptr(xv), _DTYPES[xk.dtype],
        _ptr(pos), pos0, max_pos, _ptr(q), _DTYPES[q.dtype], hq, scale, n_splits, _SCHEDULES[schedule], _ptr(out),
        _ptr(lse), _stream()), "tq_append_decode_attention_static")
    return out, lse


def dense_attention(rot: Rotation, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, seq_lens=None, max_len=None,
                    scale=None, n_splits=1, part_o=None, part_lse=None):
    """Attention over unquantised k, v [batch, n_kv_heads, capacity, 128] (fp16/fp32) as n_splits
    section partials in the packed cache's rotated domain -> (part_o, part_lse).  part_o and
    part_lse may be views of a larger partial buffer (sections after the packed ones)."""
    for x in (k, v):
        if x.dtype not in _DTYPES or not x.is_contiguous() or x.dim() != 4 or x.shape[3] != HEAD_DIM:
            raise ValueError("k and v must be contiguous [batch, n_kv_heads, capacity, 128] float16/float32")
    if k.dtype != v.dtype or k.shape != v.shape:
        raise ValueError("k and v must have the same dtype and shape")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    if k.shape[0] != bsz or k.shape[1] != rot.n_kv_heads:
        raise ValueError("k and v must be [batch, n_kv_heads, capacity, 128] for this query and rotation")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != bsz):
        raise ValueError("seq_lens must be int32 [batch]")
    cap = k.shape[2]
    if max_len is None:
        max_len = int(seq_lens.max().item()) if seq_lens is not None else cap
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    if part_o is None:
        part_o = torch.empty((n_splits, bsz, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if part_lse is None:
        part_lse = torch.empty((n_splits, bsz, hq), dtype=torch.float32, device=q.device)
    for t, shape in ((part_o, (n_splits, bsz, hq, HEAD_DIM)), (part_lse, (n_splits, bsz, hq))):
        if tuple(t.shape) != shape or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("partials must be contiguous float32 of shape %s" % (shape,))
    _check(library().tq_dense_attention(
        ctypes.byref(rot.c), _ptr(k), _ptr(v), _DTYPES[k.dtype], bsz, cap, _ptr(q), _DTYPES[q.dtype], hq,
        _ptr(seq_lens), max_len, scale, n_splits, _ptr(part_o), _ptr(part_lse), _stream()), "tq_dense_attention")
    return part_o, part_lse


def merge_splits(rot, part_o: torch.Tensor, part_lse: torch.Tensor, out=None, lse=None):
    """Log-sum-exp merge of split partials and the inverse rotation -> (out, lse).  rot=None
    merges partials of the original domain (zip_attention's) with no rotation."""
    if part_lse.dim() != 3:
        raise ValueError("part_lse must be [n_splits, batch, n_q_heads]")
    n_splits, bsz, hq = part_lse.shape
    _need(part_o, (n_splits, bsz, hq, HEAD_DIM), (torch.float32,), "part_o")
    _need(part_lse, (n_splits, bsz, hq), (torch.float32,), "part_lse")
    if out is None:
        out = torch.empty((bsz, hq, HEAD_DIM), dtype=torch.float32, device=part_o.device)
    if lse is None:
        lse = torch.empty((bsz, hq), dtype=torch.float32, device=part_o.device)
    _need(out, (bsz, hq, HEAD_DIM), (torch.float32,), "out")
    _need(lse, (bsz, hq), (torch.float32,), "lse")
    _check(library().tq_merge_splits(None if rot is None else ctypes.byref(rot.c), n_splits, bsz, hq,
                                     _ptr(part_o), _ptr(part_lse),
                                     _ptr(out), _ptr(lse), _stream()), "tq_merge_splits")
    return out, lse


def zip_store(batch: int, n_kv_heads: int, pages: int, device="cuda"):
    """Empty compressed store for one role (keys or values) -> (store uint8 [batch, n_kv_heads,
    pages, 4096], meta uint8 [batch, n_kv_heads, pages, 8])."""
    store = torch.zeros((batch, n_kv_heads, pages, ZIP_SLOT), dtype=torch.uint8, device=device)
    meta = torch.zeros((batch, n_kv_heads, pages, 8), dtype=torch.uint8, device=device)
    return store, meta


def _check_store(store, meta, batch, n_kv_heads):
    if store.dtype != torch.uint8 or store.dim() != 4 or store.shape[3] != ZIP_SLOT or not store.is_contiguous():
        raise ValueError("store must be contiguous uint8 [batch, n_kv_heads, pages, 4096]")
    if meta.dtype != torch.uint8 or tuple(meta.shape) != tuple(store.shape[:3]) + (8,) or not meta.is_contiguous():
        raise ValueError("meta must be contiguous uint8 [batch, n_kv_heads, pages, 8] matching the store")
    if store.shape[0] != batch or store.shape[1] != n_kv_heads:
        raise ValueError("store must be [batch, n_kv_heads, ...] of the BF16 buffer")


def zip_compress(x: torch.Tensor, store: torch.Tensor, meta: torch.Tensor, role: int, n_pages=None, src_page0=0,
                 dst_page0=0):
    """Compress whole 16-token pages of keys (role TQ_KEYS) or values (TQ_VALUES) x
    (bfloat16 [batch, n_kv_heads, rows, 128]): page i is rows 16 (src_page0 + i) .. +15 and
    becomes store page dst_page0 + i.  n_pages defaults to every whole page of x from
    src_page0."""
    if x.dtype != torch.bfloat16 or x.dim() != 4 or x.shape[3] != HEAD_DIM or not x.is_contiguous():
        raise ValueError("x must be contiguous bfloat16 [batch, n_kv_heads, rows, 128]")
    bsz, hkv, rows = x.shape[0], x.shape[1], x.shape[2]
    _check_store(store, meta, bsz, hkv)
    if n_pages is None:
        n_pages = rows // ZIP_PAGE - src_page0
    _check(library().tq_zip_compress(_ptr(x), role, bsz, hkv, rows, src_page0, dst_page0, n_pages, _ptr(store),
                                     _ptr(meta), store.shape[2], _stream()), "tq_zip_compress")
    return store, meta


def zip_attention(k_store, k_meta, v_store, v_meta, k_tail, v_tail, q, seq_lens=None, max_len=None, scale=None,
                  n_splits=1, out=None, lse=None, part_o=None, part_lse=None):
    """Decode attention read from compressed BF16 pages plus BF16 tail buffers (token t of a
    row past its last whole page at tail row t mod tail_rows).  n_splits == 1 -> (out, lse);
    otherwise (part_o, part_lse) in the original domain, for merge_splits(None, ...)."""
    if q.dtype not in _ZIP_Q_DTYPES or not q.is_contiguous() or q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be contiguous [batch, n_q_heads, 128] float32/float16/bfloat16")
    bsz, hq = q.shape[0], q.shape[1]
    for t in (k_tail, v_tail):
        if t.dtype != torch.bfloat16 or t.dim() != 4 or t.shape[3] != HEAD_DIM or not t.is_contiguous():
            raise ValueError("tails must be contiguous bfloat16 [batch, n_kv_heads, rows, 128]")
    if k_tail.shape != v_tail.shape or k_tail.shape[0] != bsz:
        raise ValueError("k_tail and v_tail must have the same shape [batch, n_kv_heads, rows, 128]")
    hkv = k_tail.shape[1]
    _check_store(k_store, k_meta, bsz, hkv)
    _check_store(v_store, v_meta, bsz, hkv)
    if k_store.shape != v_store.shape:
        raise ValueError("key and value stores must have the same shape")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != bsz):
        raise ValueError("seq_lens must be int32 [batch]")
    pages = k_store.shape[2]
    if max_len is None:
        max_len = int(seq_lens.max().item()) if seq_lens is not None else ZIP_PAGE * pages
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_zip_attention(
        _ptr(k_store), _ptr(k_meta), _ptr(v_store), _ptr(v_meta), pages, _ptr(k_tail), _ptr(v_tail),
        k_tail.shape[2], bsz, hkv, _ptr(q), _ZIP_Q_DTYPES[q.dtype], hq, _ptr(seq_lens), max_len, scale, n_splits,
        _ptr(out), _ptr(lse), _ptr(part_o), _ptr(part_lse), _stream()), "tq_zip_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


GTQ_ROTATION_FLOATS = 16384


def gtq_block_energies(q_cal, k_cal):
    """Block energies [n_kv_heads, 64] from calibration queries [N, n_q_heads, 128] and keys
    [N, n_kv_heads, 128] (host arrays; computed in the library on the host)."""
    import numpy as np
    q = np.ascontiguousarray(q_cal, dtype=np.float32)
    k = np.ascontiguousarray(k_cal, dtype=np.float32)
    if q.ndim != 3 or k.ndim != 3 or q.shape[0] != k.shape[0] or q.shape[2] != HEAD_DIM or k.shape[2] != HEAD_DIM:
        raise ValueError("q_cal [N, n_q_heads, 128] and k_cal [N, n_kv_heads, 128] are required")
    out = np.zeros((k.shape[1], 64), dtype=np.float32)
    _check(library().tq_gtq_block_energies(q.ctypes.data, k.ctypes.data, q.shape[0], q.shape[1], k.shape[1],
                                           out.ctypes.data), "tq_gtq_block_energies")
    return out


def gtq_allocate(energies, budget: int, b_min: int = 1, b_max: int = 4):
    """Block-GTQ greedy integer allocation (host, in the library) -> int32 bits per block."""
    import numpy as np
    e = np.ascontiguousarray(energies, dtype=np.float32)
    bits = np.zeros(e.shape[0], dtype=np.int32)
    _check(library().tq_gtq_allocate(e.ctypes.data, e.shape[0], budget, b_min, b_max, bits.ctypes.data),
           "tq_gtq_allocate")
    return bits


class GtqKeys:
    """Block-GTQ key encoders of every KV head (built on the host, held on the device).

    block_bits: int [n_kv_heads, 64] widths in 1..8 (at most four distinct per head); gauss:
    float32 [n_kv_heads, W, 128, 128] with W >= the largest width (width w of head h uses
    gauss[h, w-1]).  code_bytes: the record's code bytes for the whole cache, the largest of
    the heads' (64 when no group is wider than 4 bits)."""

    def __init__(self, block_bits, gauss, device="cuda"):
        import numpy as np
        bits = np.ascontiguousarray(block_bits, dtype=np.int32)
        g = np.ascontiguousarray(gauss, dtype=np.float32)
        hkv = bits.shape[0]
        if bits.shape != (hkv, 64) or g.ndim != 4 or g.shape[0] != hkv or g.shape[2:] != (128, 128) or \
                g.shape[1] < int(bits.max()):
            raise ValueError("block_bits [n_kv_heads, 64] and gauss [n_kv_heads, W >= max width, 128, 128] are required")
        self.heads_host = (GtqHead * hkv)()
        rot = np.zeros((hkv, GTQ_ROTATION_FLOATS), dtype=np.float32)
        for h in range(hkv):
            _check(library().tq_gtq_prepare(bits[h].ctypes.data, g[h].ctypes.data, ctypes.byref(self.heads_host[h]),
                                            rot[h].ctypes.data), "tq_gtq_prepare")
        raw = np.frombuffer(bytes(self.heads_host), dtype=np.uint8).copy()
        self.heads = torch.from_numpy(raw).to(device)
        self.rotations = torch.from_numpy(rot).to(device)
        self.n_kv_heads = hkv
        self.block_bits = bits
        self.code_bytes = max(self.heads_host[h].code_bytes for h in range(hkv))

    def n_groups(self, h):
        return self.heads_host[h].n_groups


class QjlKeys(GtqKeys):
    """Two-stage key encoders: a one-group Block-GTQ head at `bits` bits (the MSE stage,
    rotation from gauss[h, bits-1]) and the QJL projection S [n_kv_heads, 128, 128] of the
    residual, held as (S Q)^T per head.  The codes are stored bit-packed at `bits` bits per
    coordinate: 16 * bits bytes per key (code_bytes)."""

    def __init__(self, bits, gauss, S, device="cuda"):
        import numpy as np
        g = np.ascontiguousarray(gauss, dtype=np.float32)
        hkv = g.shape[0]
        sp = np.ascontiguousarray(S, dtype=np.float32)
        if sp.shape != (hkv, 128, 128):
            raise ValueError("S must be float32 [n_kv_heads, 128, 128]")
        if bits not in (1, 2, 3):
            raise ValueError("the first stage takes 1, 2 or 3 bits")
        super().__init__(np.full((hkv, 64), bits, dtype=np.int32), g, device)
        self.mse_bits = bits
        self.code_bytes = 16 * bits
        rot = self.rotations.cpu().numpy()
        proj = np.zeros((hkv, 128 * 128), dtype=np.float32)
        for h in range(hkv):
            _check(library().tq_gtq_qjl_projection(ctypes.byref(self.heads_host[h]), rot[h].ctypes.data,
                                                   sp[h].ctypes.data, proj[h].ctypes.data), "tq_gtq_qjl_projection")
        self.proj = torch.from_numpy(proj).to(device)


def gtq_quantize_keys(enc: GtqKeys, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor, pos0: int = 0):
    """Encode x [batch, n_kv_heads, n_new, 128] (fp16/fp32) into codes uint8 [batch,
    n_kv_heads, capacity, enc.code_bytes] and norms fp32 [batch, n_kv_heads, capacity, 4] at
    pos0 .."""
    if x.dtype not in _DTYPES or not x.is_contiguous() or x.dim() != 4 or x.shape[3] != HEAD_DIM:
        raise ValueError("x must be contiguous [batch, n_kv_heads, n_new, 128] float16/float32")
    bsz, hkv, n_new = x.shape[:3]
    if hkv != enc.n_kv_heads:
        raise ValueError("x has %d KV heads, the encoders %d" % (hkv, enc.n_kv_heads))
    cap = codes.shape[2]
    cb = enc.code_bytes
    if (codes.dtype != torch.uint8 or tuple(codes.shape) != (bsz, hkv, cap, cb) or not codes.is_contiguous()
            or norms.dtype != torch.float32 or tuple(norms.shape) != (bsz, hkv, cap, 4) or not norms.is_contiguous()):
        raise ValueError("codes uint8 [batch, n_kv_heads, capacity, %d] and norms float32 [.., capacity, 4]" % cb)
    _check(library().tq_gtq_quantize_keys(_ptr(enc.heads), _ptr(enc.rotations), _ptr(x), _DTYPES[x.dtype], bsz, hkv,
                                          n_new, pos0, cap, cb, _ptr(codes), _ptr(norms), _stream()),
           "tq_gtq_quantize_keys")
    return codes, norms


def gtq_attention(enc: GtqKeys, codes, norms, v, q, seq_lens=None, max_len=None, scale=None, n_splits=1, out=None,
                  lse=None, part_o=None, part_lse=None):
    """Decode attention over Block-GTQ keys and fp16 values v [batch, n_kv_heads, capacity,
    128].  n_splits == 1 -> (out, lse); otherwise (part_o, part_lse) for merge_splits(None, ..)."""
    if v.dtype != torch.float16 or not v.is_contiguous() or v.dim() != 4 or v.shape[3] != HEAD_DIM:
        raise ValueError("v must be contiguous float16 [batch, n_kv_heads, capacity, 128]")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    hkv, cap = v.shape[1], v.shape[2]
    if v.shape[0] != bsz or hkv != enc.n_kv_heads or tuple(codes.shape) != (bsz, hkv, cap, enc.code_bytes) or \
            tuple(norms.shape) != (bsz, hkv, cap, 4):
        raise ValueError("codes, norms and v must describe the same [batch, n_kv_heads, capacity] cache")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != bsz):
        raise ValueError("seq_lens must be int32 [batch]")
    if max_len is None:
        max_len = int(seq_lens.max().item()) if seq_lens is not None else cap
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_gtq_attention(
        _ptr(enc.heads), _ptr(enc.rotations), enc.code_bytes, _ptr(codes), _ptr(norms), _ptr(v), cap, bsz, hkv, _ptr(q),
        _DTYPES[q.dtype], hq, _ptr(seq_lens), max_len, scale, n_splits, _ptr(out), _ptr(lse), _ptr(part_o),
        _ptr(part_lse), _stream()), "tq_gtq_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


def gtq_append_attention(enc: GtqKeys, codes, norms, v, k_new, v_new, q, pos=None, pos0: int = 0,
                         max_pos: int = None, scale=None, n_splits=1, out=None, lse=None, part_o=None,
                         part_lse=None):
    """Append one new key/value per (sequence, KV head) at pos [batch] int32 (or pos0) to the
    Block-GTQ cache, then attend over rows ending at it, in one launch.  k_new, v_new:
    [batch, n_kv_heads, 128] of one dtype (fp16/fp32).  Returns as gtq_attention."""
    if v.dtype != torch.float16 or not v.is_contiguous() or v.dim() != 4 or v.shape[3] != HEAD_DIM:
        raise ValueError("v must be contiguous float16 [batch, n_kv_heads, capacity, 128]")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    hkv, cap = v.shape[1], v.shape[2]
    if v.shape[0] != bsz or hkv != enc.n_kv_heads or tuple(codes.shape) != (bsz, hkv, cap, enc.code_bytes) or \
            tuple(norms.shape) != (bsz, hkv, cap, 4):
        raise ValueError("codes, norms and v must describe the same [batch, n_kv_heads, capacity] cache")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x.dtype != k_new.dtype or x.dtype not in _DTYPES or not x.is_contiguous() or \
                tuple(x.shape) != (bsz, hkv, HEAD_DIM):
            raise ValueError("%s must be contiguous [batch, n_kv_heads, 128] of k_new's dtype" % name)
    if pos is not None and (pos.dtype != torch.int32 or pos.numel() != bsz):
        raise ValueError("pos must be int32 [batch]")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_gtq_append_attention(
        _ptr(enc.heads), _ptr(enc.rotations), enc.code_bytes, _ptr(codes), _ptr(norms), _ptr(v), cap, bsz, hkv, _ptr(k_new),
        _ptr(v_new), _DTYPES[k_new.dtype], _ptr(pos), pos0, max_pos, _ptr(q), _DTYPES[q.dtype], hq, scale, n_splits,
        _ptr(out), _ptr(lse), _ptr(part_o), _ptr(part_lse), _stream()), "tq_gtq_append_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


def qjl_quantize_keys(enc: QjlKeys, x: torch.Tensor, codes: torch.Tensor, norms: torch.Tensor, signs: torch.Tensor,
                      pos0: int = 0):
    """Two-stage encoding of x [batch, n_kv_heads, n_new, 128] (fp16/fp32): codes uint8
    [batch, n_kv_heads, capacity, enc.code_bytes], norms as gtq_quantize_keys (norm slot 1:
    the residual's coefficient), signs uint8 [batch, n_kv_heads, capacity, 16]."""
    if x.dtype not in _DTYPES or not x.is_contiguous() or x.dim() != 4 or x.shape[3] != HEAD_DIM:
        raise ValueError("x must be contiguous [batch, n_kv_heads, n_new, 128] float16/float32")
    bsz, hkv, n_new = x.shape[:3]
    cap = codes.shape[2]
    cb = enc.code_bytes
    if hkv != enc.n_kv_heads or tuple(codes.shape) != (bsz, hkv, cap, cb) or codes.dtype != torch.uint8 or \
            tuple(norms.shape) != (bsz, hkv, cap, 4) or norms.dtype != torch.float32 or \
            tuple(signs.shape) != (bsz, hkv, cap, 16) or signs.dtype != torch.uint8 or \
            not (codes.is_contiguous() and norms.is_contiguous() and signs.is_contiguous()):
        raise ValueError("codes uint8 [b, kv, cap, %d], norms float32 [b, kv, cap, 4], signs uint8 [b, kv, cap, 16]"
                         % cb)
    _check(library().tq_gtq_qjl_quantize_keys(_ptr(enc.heads), _ptr(enc.rotations), _ptr(enc.proj), enc.mse_bits,
                                              _ptr(x),
                                              _DTYPES[x.dtype], bsz, hkv, n_new, pos0, cap, _ptr(codes),
                                              _ptr(norms), _ptr(signs), _stream()), "tq_gtq_qjl_quantize_keys")


def qjl_attention(enc: QjlKeys, codes, norms, signs, v, q, seq_lens=None, max_len=None, scale=None, n_splits=1,
                  out=None, lse=None, part_o=None, part_lse=None):
    """Decode attention over two-stage keys and fp16 values; returns as gtq_attention."""
    if v.dtype != torch.float16 or not v.is_contiguous() or v.dim() != 4 or v.shape[3] != HEAD_DIM:
        raise ValueError("v must be contiguous float16 [batch, n_kv_heads, capacity, 128]")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    hkv, cap = v.shape[1], v.shape[2]
    if v.shape[0] != bsz or hkv != enc.n_kv_heads or tuple(codes.shape) != (bsz, hkv, cap, enc.code_bytes) or \
            tuple(norms.shape) != (bsz, hkv, cap, 4) or tuple(signs.shape) != (bsz, hkv, cap, 16):
        raise ValueError("codes, norms, signs and v must describe the same [batch, n_kv_heads, capacity] cache")
    if seq_lens is not None and (seq_lens.dtype != torch.int32 or seq_lens.numel() != bsz):
        raise ValueError("seq_lens must be int32 [batch]")
    if max_len is None:
        max_len = int(seq_lens.max().item()) if seq_lens is not None else cap
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_gtq_qjl_attention(
        _ptr(enc.heads), _ptr(enc.rotations), _ptr(enc.proj), enc.mse_bits, _ptr(codes), _ptr(norms), _ptr(signs),
        _ptr(v), cap,
        bsz, hkv, _ptr(q), _DTYPES[q.dtype], hq, _ptr(seq_lens), max_len, scale, n_splits, _ptr(out), _ptr(lse),
        _ptr(part_o), _ptr(part_lse), _stream()), "tq_gtq_qjl_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)


def qjl_append_attention(enc: QjlKeys, codes, norms, signs, v, k_new, v_new, q, pos=None, pos0: int = 0,
                         max_pos: int = None, scale=None, n_splits=1, out=None, lse=None, part_o=None,
                         part_lse=None):
    """gtq_append_attention for two-stage keys: the new key's codes, norm, sign bits and
    coefficient and its value written at pos (or pos0), then attention, in one launch."""
    if v.dtype != torch.float16 or not v.is_contiguous() or v.dim() != 4 or v.shape[3] != HEAD_DIM:
        raise ValueError("v must be contiguous float16 [batch, n_kv_heads, capacity, 128]")
    if q.dtype not in _DTYPES or not q.is_contiguous():
        raise ValueError("q must be a contiguous float16/float32 tensor")
    if q.dim() != 3 or q.shape[2] != HEAD_DIM:
        raise ValueError("q must be [batch, n_q_heads, 128]")
    bsz, hq = q.shape[0], q.shape[1]
    hkv, cap = v.shape[1], v.shape[2]
    if v.shape[0] != bsz or hkv != enc.n_kv_heads or tuple(codes.shape) != (bsz, hkv, cap, enc.code_bytes) or \
            tuple(norms.shape) != (bsz, hkv, cap, 4) or tuple(signs.shape) != (bsz, hkv, cap, 16):
        raise ValueError("codes, norms, signs and v must describe the same [batch, n_kv_heads, capacity] cache")
    for name, x in (("k_new", k_new), ("v_new", v_new)):
        if x.dtype != k_new.dtype or x.dtype not in _DTYPES or not x.is_contiguous() or \
                tuple(x.shape) != (bsz, hkv, HEAD_DIM):
            raise ValueError("%s must be contiguous [batch, n_kv_heads, 128] of k_new's dtype" % name)
    if pos is not None and (pos.dtype != torch.int32 or pos.numel() != bsz):
        raise ValueError("pos must be int32 [batch]")
    if max_pos is None:
        max_pos = int(pos.max().item()) if pos is not None else pos0
    if scale is None:
        scale = 1.0 / math.sqrt(HEAD_DIM)
    out, lse, part_o, part_lse = _outputs(n_splits, bsz, hq, q.device, out, lse, part_o, part_lse)
    _check(library().tq_gtq_qjl_append_attention(
        _ptr(enc.heads), _ptr(enc.rotations), _ptr(enc.proj), enc.mse_bits, _ptr(codes), _ptr(norms), _ptr(signs),
        _ptr(v), cap,
        bsz, hkv, _ptr(k_new), _ptr(v_new), _DTYPES[k_new.dtype], _ptr(pos), pos0, max_pos, _ptr(q), _DTYPES[q.dtype],
        hq, scale, n_splits, _ptr(out), _ptr(lse), _ptr(part_o), _ptr(part_lse), _stream()),
        "tq_gtq_qjl_append_attention")
    return (out, lse) if n_splits == 1 else (part_o, part_lse)

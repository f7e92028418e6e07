"""Seeded synthetic decode-attention workloads (shared input generator).

This module is the only thing the oracle and the HIP path both consume.  It draws random
numbers (query/key/value activations, outlier channels, per-channel scales, the +-1 sign
flips and the SO(4) quaternion pairs of the rotation) and holds none of the method's
arithmetic.  Shapes and distributions follow the workloads the pages measure on: a 4B
GQA model at 8K context ("TurboQuant ... MNN on phones", section 4), 128K-token decode
("RoPE-Aware Bit Allocation for KV-Cache Quantization", deployment results) and 32K
contexts with the IsoQuant rotation ("RotaryQuant ...", key findings) and a BF16 8B GQA
model at 8K context, batch 32, for the lossless exponent codec ("ZipFusion ...",
experiments: Llama 3.1 8B / Qwen3-8B, 8192-token prompts).  No dataset is read; Gaussian
activations with outlier channels stand in for real model activations.
"""

import os
from dataclasses import dataclass, replace

import numpy as np

HEAD_DIM = 128


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    seq_len: int
    bits_k: int
    bits_v: int
    group: int               # rotation block = norm group = codebook dimension
    so4: bool                # compose the Hadamard with SO(4) block rotations
    dtype: str               # "float32", "float16" or "bfloat16" activations (bfloat16 as uint16 bits)
    outliers: str            # "fixed2x10", "seeded4x8" or "lognormal"
    n_splits: int = 1        # key-axis splits used when the workload is timed
    scale: float = HEAD_DIM ** -0.5
    codec: str = "turboquant"  # "turboquant" (packed 3/4-bit codes) or "zip" (lossless BF16 pages)

    @property
    def group_size(self):
        return self.n_q_heads // self.n_kv_heads

    def with_len(self, seq_len, batch=None):
        return replace(self, seq_len=seq_len, batch=self.batch if batch is None else batch)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 1, 256, 3, 3, 32, False, "float32", "fixed2x10"),
    "gqa8k": Workload("gqa8k", 1, 32, 8, 8192, 3, 3, 32, False, "float16", "seeded4x8", n_splits=32),
    "batched": Workload("batched", 32, 32, 8, 4096, 4, 3, 32, False, "float16", "seeded4x8", n_splits=2),
    "long128k": Workload("long128k", 1, 16, 2, 131072, 3, 3, 32, False, "float16", "lognormal",
                         n_splits=64),
    "isoquant32k": Workload("isoquant32k", 8, 32, 8, 32768, 3, 3, 128, True, "float16", "seeded4x8",
                            n_splits=8),
    # 8192-token prompt in compressed pages plus 8 generated tokens in the open page; the
    # bits, group and so4 fields do not apply to the lossless codec
    # Block-GTQ keys at a 3-bit average budget (192 bits over 64 RoPE blocks, widths 1..4)
    # with fp16 values; log-normal channel scales give the blocks unequal energies
    "gtq32k": Workload("gtq32k", 4, 32, 8, 32768, 3, 16, 128, False, "float16", "lognormal", n_splits=8,
                       codec="gtq"),
    # two-stage keys at 2 bits (1-bit MSE + 1-bit QJL residual), fp16 values
    "qjl32k": Workload("qjl32k", 4, 32, 8, 32768, 2, 16, 128, False, "float16", "lognormal", n_splits=8,
                       codec="qjl"),
    "zipfusion8k": Workload("zipfusion8k", 32, 32, 8, 8200, 16, 16, 128, False, "bfloat16", "seeded4x8",
                            n_splits=1, codec="zip"),
}


def bf16_bits(x):
    """float32 array -> BF16 bit patterns (uint16), rounded to nearest even: how a BF16
    model stores its activations.  Input preparation only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def _stream_normals(seed_seq, bsz, hkv, t, fill):
    """Draw K or V as one independent N(0, 1) stream per (sequence, KV head), on threads.

    fill(b, kv, x) receives the float32 [t, 128] draw of that stream and stores it.  Each
    stream has its own spawned seed, so the result does not depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor

    seeds = seed_seq.spawn(bsz * hkv)

    def one(i):
        b, kv = divmod(i, hkv)
        fill(b, kv, np.random.default_rng(seeds[i]).standard_normal((t, HEAD_DIM), dtype=np.float32))

    with ThreadPoolExecutor(max_workers=max(1, min(16, len(seeds), os.cpu_count() or 1))) as ex:
        list(ex.map(one, range(len(seeds))))


def generate(w: Workload, seed: int = 0, with_kv: bool = True):
    """Draw one workload's inputs.

    Returns a dict of numpy arrays:
      q [B, Hq, 128], k [B, Hkv, T, 128], v [B, Hkv, T, 128] in ``w.dtype`` (bfloat16 as
      uint16 bit patterns);
      signs [Hkv, 128] float32 (+-1); so4 [Hkv, 32, 2, 4] float32 unit (q_L, q_R) or None;
      seq_lens [B] int32 (all equal to T).
    Every array has its own random stream (K and V one per (sequence, KV head)).
    """
    ss = np.random.SeedSequence(seed)
    s_q, s_k, s_v, s_sign, s_so4, s_ch, s_sk, s_sv = ss.spawn(8)
    bsz, hq, hkv, t = w.batch, w.n_q_heads, w.n_kv_heads, w.seq_len
    g = w.group_size
    bf16 = w.dtype == "bfloat16"
    dt = np.float16 if w.dtype == "float16" else np.uint16 if bf16 else np.float32
    cast = bf16_bits if bf16 else (lambda a: a)

    # per-(KV head, channel) multipliers shared by K and that head's queries, and for V
    mul_k = np.ones((hkv, HEAD_DIM), np.float32)
    mul_v = np.ones((hkv, HEAD_DIM), np.float32)
    if w.outliers == "fixed2x10":
        # channels 3 and 77 scaled by 10 in q, K and V
        mul_k[:, [3, 77]] = 10.0
        mul_v[:, [3, 77]] = 10.0
    elif w.outliers == "seeded4x8":
        # 4 seeded channels per KV head scaled by 8 in K, V and that head's queries
        r_ch = np.random.default_rng(s_ch)
        for kv in range(hkv):
            ch = r_ch.choice(HEAD_DIM, size=4, replace=False)
            mul_k[kv, ch] = 8.0
            mul_v[kv, ch] = 8.0
    elif w.outliers == "lognormal":
        # per-(KV head, channel) scale e^z, z ~ N(0, 1): one draw shared by K and its
        # queries, an independent draw for V
        mul_k = np.exp(np.random.default_rng(s_sk).standard_normal((hkv, HEAD_DIM))).astype(np.float32)
        mul_v = np.exp(np.random.default_rng(s_sv).standard_normal((hkv, HEAD_DIM))).astype(np.float32)
    else:
        raise ValueError(w.outliers)

    q = np.random.default_rng(s_q).standard_normal((bsz, hq, HEAD_DIM), dtype=np.float32)
    q *= np.repeat(mul_k, g, axis=0)[None]
    k = v = None
    if with_kv:
        k = np.empty((bsz, hkv, t, HEAD_DIM), dt)
        v = np.empty((bsz, hkv, t, HEAD_DIM), dt)

        def fill_k(b, kv, x):
            k[b, kv] = cast(x * mul_k[kv])

        def fill_v(b, kv, x):
            v[b, kv] = cast(x * mul_v[kv])

        _stream_normals(s_k, bsz, hkv, t, fill_k)
        _stream_normals(s_v, bsz, hkv, t, fill_v)

    r_sign = np.random.default_rng(s_sign)
    signs = np.where(r_sign.random((hkv, HEAD_DIM)) < 0.5, -1.0, 1.0).astype(np.float32)
    so4 = None
    if w.so4:
        quat = np.random.default_rng(s_so4).standard_normal((hkv, HEAD_DIM // 4, 2, 4))
        so4 = (quat / np.linalg.norm(quat, axis=-1, keepdims=True)).astype(np.float32)
    extra = {}
    if w.codec == "gtq":
        # a calibration prefix of queries and keys (same laws) for the block energies, and a
        # Gaussian matrix per (KV head, width) from which each group's random rotation is drawn
        s_cq, s_ck, s_rot = ss.spawn(3)
        n_cal = 256
        q_cal = np.random.default_rng(s_cq).standard_normal((n_cal, hq, HEAD_DIM), dtype=np.float32)
        q_cal *= np.repeat(mul_k, g, axis=0)[None]
        k_cal = np.random.default_rng(s_ck).standard_normal((n_cal, hkv, HEAD_DIM), dtype=np.float32)
        k_cal *= mul_k[None]
        # widths 5-8 (byte containers) draw from a stream of their own, so that widths 1-4
        # keep their matrices
        (s_rot_wide,) = ss.spawn(1)
        gauss = np.concatenate(
            [np.random.default_rng(s_rot).standard_normal((hkv, 4, HEAD_DIM, HEAD_DIM), dtype=np.float32),
             np.random.default_rng(s_rot_wide).standard_normal((hkv, 4, HEAD_DIM, HEAD_DIM), dtype=np.float32)], axis=1)
        extra = {"q_cal": q_cal, "k_cal": k_cal, "gauss": gauss}
    if w.codec == "qjl":
        # per KV head: Gaussian matrices for the MSE stage's rotation (as Block-GTQ's) and
        # the residual's projection S (m = 128 rows)
        s_rot, s_proj = ss.spawn(2)
        extra = {"gauss": np.random.default_rng(s_rot).standard_normal((hkv, 4, HEAD_DIM, HEAD_DIM), dtype=np.float32),
                 "proj": np.random.default_rng(s_proj).standard_normal((hkv, HEAD_DIM, HEAD_DIM), dtype=np.float32)}
    return {
        **extra,
        "q": bf16_bits(q) if bf16 else q.astype(dt),
        "k": k,
        "v": v,
        "signs": signs,
        "so4": so4,
        "seq_lens": np.full(bsz, t, dtype=np.int32),
    }

// HIP kernels of the lossless BF16 exponent codec of a KV cache and of decode attention
// read straight from the compressed pages.  Target: gfx950 (MI355X), wave64.
//
// Method source: "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient
// LLM Decoding" (paper-daily.com): the compression format (only the exponent is coded: a
// chunk of 512 values keeps every low byte and replaces the rest by a 4-bit sign + exponent
// offset code against the chunk's even base b, when all exponents lie in [b, b + 15]), the
// page layout (16-token pages, 4 key and 4 value chunks per page and head, 8 bytes of
// metadata each), the register decode (the high byte of a value is sign * 128 + b/2 + d:
// one 32-bit add of b/2 in every byte yields four high bytes, with no rounding) and the
// fused operator (pages staged on chip still compressed; each thread decodes the 8 values
// it feeds the matrix unit, keys and values laid out for their own products).
//
// Layout of one (sequence, KV head) stream:
//   store [page][4096 bytes]: the page's 4 chunks back to back from the slot start, each
//     either coded (512 low bytes, then 256 code bytes) or kept (its 512 BF16 values); the
//     rest of the slot is zero.  Keys: chunk c is the page's tokens 4c .. 4c+3, token-major
//     (a group of 8 values = 8 coordinates of one token).  Values: chunk c is coordinates
//     32c .. 32c+31 of the page's 16 tokens, coordinate-major (a group = 8 tokens of one
//     coordinate).
//   meta [page][8 bytes]: little-endian u32 byte offset of the page's first chunk in the
//     stream, then one byte per chunk: 0xFF for a kept chunk, else b/2.
//   Code byte 4g + j of a chunk holds value 8g + j (sign bit 7, d bits 0-2) and value
//     8g + j + 4 (sign bit 6, d bits 3-5), d = (exponent - b) / 2 rounded down.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2z = 0.69314718055994531f;
constexpr uint32_t kKept = 0xFFFFFFFFu;  // decode mode of a kept (uncompressed) chunk
constexpr float kRescale = 8.f;          // log2 headroom of the lazily updated softmax reference

__device__ __forceinline__ int wave_min(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = min(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// ---------------------------------------------------------------------------------------
// Compression of whole pages.  One workgroup per (page, KV head, sequence): the page's 16
// tokens are staged in LDS; wave c codes chunk c; lane l takes the chunk's group l (values
// 8l .. 8l + 7 in chunk order: for keys 8 coordinates of one token, for values 8 tokens of
// one coordinate).
__global__ __launch_bounds__(256) void zip_compress_kernel(const ZipCompressArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kZipPage * kHeadDim];
  __shared__ uint32_t flag[4];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, c = tid >> 6;
  const size_t stream = (size_t)b * a.n_kv_heads + h;
  const uint16_t* src = a.x + (stream * a.x_rows + (size_t)kZipPage * (a.src_page0 + i)) * kHeadDim;
  *(uint4*)(tile + 8 * tid) = *(const uint4*)(src + 8 * tid);
  __syncthreads();
  uint32_t wd[4];  // the group's 8 values, two per word (the first in the low half)
  if (a.values) {
    const int d = 32 * c + (lane >> 1), t0 = 8 * (lane & 1);
#pragma unroll
    for (int k = 0; k < 4; ++k)
      wd[k] = (uint32_t)tile[(t0 + 2 * k) * kHeadDim + d] | ((uint32_t)tile[(t0 + 2 * k + 1) * kHeadDim + d] << 16);
  } else {
    const uint4 w = *(const uint4*)(tile + 512 * c + 8 * lane);
    wd[0] = w.x;
    wd[1] = w.y;
    wd[2] = w.z;
    wd[3] = w.w;
  }
  uint32_t v[8];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] = wd[k] & 0xFFFFu;
    v[2 * k + 1] = wd[k] >> 16;
  }
  int mn = 255, mx = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int e = (v[k] >> 7) & 0xFF;
    mn = min(mn, e);
    mx = max(mx, e);
  }
  const int base = wave_min(mn) & ~1;  // the chunk's smallest exponent, rounded down to even
  const bool coded = wave_max(mx) - base <= 15;
  if (lane == 0) flag[c] = coded ? (uint32_t)(base >> 1) : 0xFFu;
  __syncthreads();
  uint32_t off = 0, total = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sz = flag[j] == 0xFFu ? 1024u : 768u;
    off += j < c ? sz : 0u;
    total += sz;
  }
  uint8_t* dst = a.store + (stream * a.store_pages + a.dst_page0 + i) * kZipSlot;
  if (coded) {
    // low bytes of the 8 values (bytes 0 and 2 of each word)
    const uint32_t lo0 = __builtin_amdgcn_perm(wd[1], wd[0], 0x06040200u);
    const uint32_t lo1 = __builtin_amdgcn_perm(wd[3], wd[2], 0x06040200u);
    uint32_t codes = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t s1 = v[j] >> 15, d1 = (((v[j] >> 7) & 0xFF) - base) >> 1;
      const uint32_t s5 = v[j + 4] >> 15, d5 = (((v[j + 4] >> 7) & 0xFF) - base) >> 1;
      codes |= ((s1 << 7) | d1 | (s5 << 6) | (d5 << 3)) << (8 * j);
    }
    *(u32x2*)(dst + off + 8 * lane) = u32x2{lo0, lo1};
    *(uint32_t*)(dst + off + 512 + 4 * lane) = codes;
  } else {
    *(uint4*)(dst + off + 16 * lane) = make_uint4(wd[0], wd[1], wd[2], wd[3]);
  }
  // the slot's unused bytes (total is a multiple of 256)
  if ((uint32_t)(16 * tid) >= total) *(uint4*)(dst + 16 * tid) = make_uint4(0, 0, 0, 0);
  if (tid == 0) {
    const uint32_t start = (uint32_t)(a.dst_page0 + i) * (uint32_t)kZipSlot;
    *(u32x2*)(a.meta + (stream * a.store_pages + a.dst_page0 + i) * 8) =
        u32x2{start, flag[0] | (flag[1] << 8) | (flag[2] << 16) | (flag[3] << 24)};
  }
}

// ---------------------------------------------------------------------------------------
// Register decode of one coded group straight into a matrix-unit operand: 8 BF16 values,
// two per word in order.  The high bytes of values 1-4 are the code word masked with
// 0x87878787 plus b/2 in every byte; those of values 5-8 the code word shifted into the same
// places plus b/2.  A byte permute then pairs each high byte with its low byte.
__device__ __forceinline__ u32x4 decode_group(u32x2 lo, uint32_t code, uint32_t bh4) {
  const uint32_t h1 = (code & 0x87878787u) + bh4;
  const uint32_t h5 = (((code >> 3) & 0x07070707u) | ((code << 1) & 0x80808080u)) + bh4;
  return u32x4{__builtin_amdgcn_perm(h1, lo.x, 0x05010400u), __builtin_amdgcn_perm(h1, lo.x, 0x07030602u),
               __builtin_amdgcn_perm(h5, lo.y, 0x05010400u), __builtin_amdgcn_perm(h5, lo.y, 0x07030602u)};
}

// Byte offset of chunk c from its page start and its decode mode (kKept, or b/2 in every
// byte), from the page's four chunk flags.
__device__ __forceinline__ void chunk_at(uint32_t flags, int c, uint32_t& off, uint32_t& mode) {
  off = 768u * (uint32_t)c;
#pragma unroll
  for (int j = 0; j < 3; ++j) off += (j < c && ((flags >> (8 * j)) & 0xFFu) == 0xFFu) ? 256u : 0u;
  const uint32_t f = (flags >> (8 * c)) & 0xFFu;
  mode = f == 0xFFu ? kKept : (f & 0x7Fu) * 0x01010101u;
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float x, float y) {
  return __builtin_bit_cast(uint32_t, bf16x2{(__bf16)x, (__bf16)y});
}
// x = hi + lo with hi, lo BF16 (round to nearest even): hi + lo carries 16 significant bits
__device__ __forceinline__ float bf16_lo(float x) { return x - (float)(__bf16)x; }

// kept ? raw : coded, word by word (a bit select, no branch)
__device__ __forceinline__ u32x4 pick(bool kept, u32x4 raw, u32x4 coded) {
  const uint32_t m = kept ? 0xFFFFFFFFu : 0u;
  return (raw & m) | (coded & ~m);
}

template <typename T>
__device__ __forceinline__ T lds_read(const uint8_t* p) {
  return *(const T*)p;
}

// Attention of one (sequence, KV head, section, head slice of up to 8 heads) over its
// tokens, on the matrix unit.  The section's pages go to the waves in turn; each wave
// streams its pages through its own ring of D LDS stages (a stage: the page's keys, then
// its values, 4 KB each) with direct global -> LDS copies of exactly the stored bytes, the
// metadata of the page D stages ahead riding along, so the copies in flight cost no
// registers and several pages per wave are in flight while one is computed.
//
// Per page, with bf16 16x16x32 products:
//   scores S[token][col] = K (16 tokens x 32 coordinates, a key group per lane) x Q (32 x 16)
//     over 4 coordinate blocks.  Columns are (part, head): the query in BF16 as hi + lo,
//     heads in columns 0-7 (hi) and 8-15 (lo); a lane exchange adds the two parts.  Lane l
//     ends up with tokens 4 (l >> 4) .. + 3 of the page for its column.
//   output O[col][coord] += P (16 x 32) x V (32 x 16 coordinates) for 8 coordinate tiles:
//     the weights as BF16 hi + lo in rows 0-7 and 8-15, straight from the lanes' score
//     registers, in k slots 8 (l >> 4) .. + 3; slots + 4 .. + 7 carry zero weight.  The value
//     operand of those 4 tokens is half a value group (8 tokens of one coordinate).
// The softmax reference m is updated lazily (only when a score exceeds it by 8 in log2
// units), so that weights stay in (0, 256]; each wave keeps its own m, sum and output,
// merged across waves at the end.  Results are in the original domain.
template <int NW, int D, int QT>
__global__ __launch_bounds__(64 * NW) void zip_attention_kernel(const ZipAttnArgs a) {
  constexpr int STAGE = 2 * kZipSlot;  // the page's keys, then its values
  constexpr int MSLOT = 256;           // one stage's metadata (16 bytes used)
  constexpr int WAVE_LDS = D * STAGE + 2 * D * MSLOT;
  constexpr int NDMA = 9;              // copies per stage: 2 pages x 4, and the metadata
  static_assert(D >= 2 && D * NDMA <= 63, "ring depth within the memory counter");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NW * WAVE_LDS];
  __shared__ float part_m[NW][8], part_l[NW][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, in a scalar register
  const int unit = blockIdx.x / a.n_slices, slice = blockIdx.x - unit * a.n_slices;
  const int split = unit % a.n_splits, kv = (unit / a.n_splits) % a.n_kv_heads;
  const int b = unit / (a.n_splits * a.n_kv_heads);
  const int h0 = kv * a.group_size + slice * a.heads_per_slice;
  const int hs = min(a.heads_per_slice, a.group_size - slice * a.heads_per_slice);
  // lengths beyond max_len (checked against the store and the tail on the host) are clamped
  const int T = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_len)) : a.max_len;
  const int full = min(T >> 4, a.store_pages);  // pages read from the store
  // sections of whole pages
  const int C = (((T + a.n_splits - 1) / a.n_splits) + 15) & ~15;
  const int lo = min(T, split * C), hi = min(T, lo + C);
  const int pg_lo = lo >> 4, pg_hi = (hi + 15) >> 4;
  const int npages = lo < hi ? pg_hi - pg_lo : 0;  // an empty section (lo = hi = T) has none
  const int n = npages > wv ? (npages - wv + NW - 1) / NW : 0;  // this wave's pages

  const size_t stream = (size_t)b * a.n_kv_heads + kv;
  const uint8_t* ks = a.k_store + stream * a.store_pages * kZipSlot;
  const uint8_t* vs = a.v_store + stream * a.store_pages * kZipSlot;
  const uint8_t* km = a.k_meta + stream * a.store_pages * 8;
  const uint8_t* vm = a.v_meta + stream * a.store_pages * 8;
  const uint8_t* kt = (const uint8_t*)(a.k_tail + stream * a.tail_rows * kHeadDim);
  const uint8_t* vt = (const uint8_t*)(a.v_tail + stream * a.tail_rows * kHeadDim);
  // a start offset is trusted only as far as a whole page slot stays inside the stream
  const uint32_t lim = (uint32_t)max(a.store_pages - 1, 0) * (uint32_t)kZipSlot;

  uint8_t* wlds = lds + wv * WAVE_LDS;  // this wave's ring, then its metadata slots
  uint8_t* mlds = wlds + D * STAGE;
  const uint32_t wlds_a = lds_addr(wlds), mlds_a = lds_addr(mlds);

  auto page_of = [&](int s) { return pg_lo + wv + NW * s; };
  // metadata of stage s (keys: start, flags; values: start, flags) into slot s mod 2D;
  // words of pages outside the store are copied from a valid dummy address
  auto meta_dma = [&](int s) {
    const int p = page_of(s);
    const uint8_t* m = (lane & 2) ? vm : km;
    const void* src = (lane < 4 && p < full) ? (const void*)(m + (size_t)p * 8 + 4 * (lane & 1)) : (const void*)kt;
    lds_dma_addr<4, false>(mlds_a + (s % (2 * D)) * MSLOT, src);
  };
  // one 4 KB page region of a stage: `bytes` from `src`; lanes past them copy the first
  // 16 bytes again (into the region's unused part), so every stage issues the same copies
  auto page_dma = [&](uint32_t dst, const uint8_t* src, uint32_t bytes) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t o = 1024u * k + 16u * lane;
      lds_dma<16, true>(dst + 1024u * k, src, o < bytes ? o : 0u);
    }
  };
  auto page_bytes = [&](uint32_t flags) {
    uint32_t nb = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) nb += ((flags >> (8 * j)) & 0xFFu) == 0xFFu ? 1024u : 768u;
    return nb;
  };
  // stage s: a stored page compressed, or the open page from the tail buffer; then the
  // metadata of stage s + D
  auto issue = [&](int s) {
    const int p = page_of(s);
    const u32x4 m = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT);
    lds_wait();
    const uint32_t dst = wlds_a + (s % D) * STAGE;
    if (p < full) {
      page_dma(dst, ks + min(__builtin_amdgcn_readfirstlane(m.x) & ~15u, lim),
               page_bytes(__builtin_amdgcn_readfirstlane(m.y)));
      page_dma(dst + kZipSlot, vs + min(__builtin_amdgcn_readfirstlane(m.z) & ~15u, lim),
               page_bytes(__builtin_amdgcn_readfirstlane(m.w)));
    } else {
      const size_t row = (size_t)((16 * p) % a.tail_rows) * 256;
      page_dma(dst, kt + row, kZipSlot);
      page_dma(dst + kZipSlot, vt + row, kZipSlot);
    }
    meta_dma(s + D);
  };

  // prologue: the first D stages' metadata; the query as matrix operands (BF16 hi in
  // columns 0-7, lo in 8-15; lane l holds column l & 15, coordinates 32 kb + 8 (l >> 4) ..)
  for (int s = 0; s < D; ++s)
    if (s < n) meta_dma(s);
  u32x4 qf[4];
  {
    const int col = lane & 15, hh = col & 7;
    const bool live = hh < hs;
    const size_t qrow = ((size_t)b * a.n_q_heads + h0 + (live ? hh : 0)) * kHeadDim;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      float x[8];
      const int d0 = 32 * kb + 8 * (lane >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (QT == 1) x[e] = (float)((const _Float16*)a.q)[qrow + d0 + e];
        else if (QT == 2) x[e] = __uint_as_float((uint32_t)((const uint16_t*)a.q)[qrow + d0 + e] << 16);
        else x[e] = ((const float*)a.q)[qrow + d0 + e];
        if (!live) x[e] = 0.f;
        if (col >= 8) x[e] = bf16_lo(x[e]);
      }
      qf[kb] = u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
    }
  }
  // every ordinary load has returned here (the compiler waits for all copies with them)
  asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]));
  vm_wait<0>();
  for (int s = 0; s < D; ++s)
    if (s < n) issue(s);

  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, thr = -INFINITY, lsum = 0.f;
  const int col = lane & 15;
  const int jr = lane >> 4;  // row group: score rows (tokens) 4 jr .. 4 jr + 3

  for (int s = 0; s < n; ++s) {
    const int younger = min(D - 1, n - 1 - s);
    if (younger >= 3) vm_wait<3 * NDMA>();
    else if (younger == 2) vm_wait<2 * NDMA>();
    else if (younger == 1) vm_wait<NDMA>();
    else vm_wait<0>();
    const int p = page_of(s);
    const bool stored = p < full;
    const int np = min(16, hi - 16 * p);  // the page's tokens in the section
    const u32x4 m = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT);
    const uint32_t kflags = stored ? __builtin_amdgcn_readfirstlane(m.y) : kKept;
    const uint32_t vflags = __builtin_amdgcn_readfirstlane(m.w);
    const uint8_t* sb = wlds + (s % D) * STAGE;

    // ---- operand reads, all issued before any use (branch-free: a kept key group is one
    // 16-byte word, a coded one 8 low bytes and a code word; both are read, the mode picks)
    u32x4 kraw[4];
    uint32_t kcode[4], kmode;
    {
      const int i = col & 3;  // key operand row = token col: chunk col >> 2, row i in it
      uint32_t off;
      chunk_at(kflags, col >> 2, off, kmode);
      const bool kept = kmode == kKept;
      const uint8_t* cw = sb + off + (kept ? 256 * i : 128 * i);
      const uint8_t* cc = sb + off + 512 + 64 * i;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int g = 4 * kb + jr;  // group of the token: coordinates 8g .. 8g + 7
        kraw[kb] = lds_read<u32x4>(cw + (kept ? 16 * g : 8 * g));
        kcode[kb] = lds_read<uint32_t>(cc + 4 * g);
      }
    }
    // value operand of coordinate 16 ct + col, tokens 4 jr .. + 3: half (jr & 1) of group
    // (coordinate, tokens 8 (jr >> 1) .. + 7)
    u32x2 vraw[8];
    uint32_t vcode[8], vmode[8];
    const int half = jr & 1;
    if (stored) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        uint32_t off, mode;
        chunk_at(vflags, ct >> 1, off, mode);
        const int g = 2 * (16 * (ct & 1) + col) + (jr >> 1);
        vmode[ct] = mode;
        vraw[ct] = mode == kKept ? lds_read<u32x2>(sb + kZipSlot + off + 16 * g + 8 * half)
                                 : u32x2{lds_read<uint32_t>(sb + kZipSlot + off + 8 * g + 4 * half), 0u};
        vcode[ct] = lds_read<uint32_t>(sb + kZipSlot + off + 512 + 4 * g);
      }
    } else {
      // the open page, token-major BF16; tokens past the row are zeros
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int d = 16 * ct + col;
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * jr + e;
          w[e] = t < np ? (uint32_t)lds_read<uint16_t>(sb + kZipSlot + 256 * t + 2 * d) : 0u;
        }
        vmode[ct] = kKept;
        vraw[ct] = u32x2{w[0] | (w[1] << 16), w[2] | (w[3] << 16)};
        vcode[ct] = 0u;
      }
    }

    // ---- scores of the page's 16 tokens
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 dec = decode_group(u32x2{kraw[kb].x, kraw[kb].y}, kcode[kb], kmode);
      sc = mfma_bf16(pick(kmode == kKept, kraw[kb], dec), qf[kb], sc);
    }
    // hi + lo parts, scale, mask; this lane's rows are tokens 4 jr + e
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = (sc[e] + dpp<0x128>(sc[e])) * a.scale_log2;
      x[e] = 4 * jr + e < np ? v : -INFINITY;
      bm = fmaxf(bm, x[e]);
    }
    bm = max_rows(bm);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(bm > thr) != 0, 0)) {
      const float mnew = fmaxf(mref, bm);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);  // 0 on the first page
      lsum *= alpha;
      // output rows 4 jr + e are (part, head) (4 jr + e) & 7: that head's factor
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float al = __shfl(alpha, (4 * jr + e) & 7);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct][e] *= al;
      }
      mref = mnew;
      thr = mnew + kRescale;
    }
    // weights: BF16 hi (columns 0-7) or lo (8-15) parts in k slots 8 jr .. + 3
    u32x4 pf;
    {
      float pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = __builtin_amdgcn_exp2f(x[e] - mref);
        lsum += pw[e];
        if (col >= 8) pw[e] = bf16_lo(pw[e]);
      }
      pf = u32x4{pack_bf16(pw[0], pw[1]), pack_bf16(pw[2], pw[3]), 0u, 0u};
    }

    // ---- output: 8 coordinate tiles
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      // coded: the half's 4 high bytes (values 1-4 or 5-8 of the group: the signs in bit 7
      // or 6, the offsets in bits 0-2 or 3-5) plus b/2, paired byte by byte with its low
      // word; kept: the two raw words, passed through by the same permutes
      const bool kept = vmode[ct] == kKept;
      const uint32_t c = vcode[ct];
      const uint32_t hb = (((c >> (3 * half)) & 0x07070707u) | ((c << half) & 0x80808080u)) + vmode[ct];
      const uint32_t H = kept ? vraw[ct].y : hb;
      const uint32_t w0 = __builtin_amdgcn_perm(H, vraw[ct].x, kept ? 0x03020100u : 0x05010400u);
      const uint32_t w1 = __builtin_amdgcn_perm(H, vraw[ct].x, kept ? 0x07060504u : 0x07030602u);
      acc[ct] = mfma_bf16(pf, u32x4{w0, w1, 0u, 0u}, acc[ct]);
    }
    // the stage's slot is refilled with stage s + D once its reads are done
    if (s + D < n) {
      lds_wait();
      issue(s + D);
    }
  }

  // ---- merge the waves: sums over the row groups, hi + lo output rows
  vm_wait<0>();
  lsum = sum_rows(lsum);
  __syncthreads();  // every wave is done with its ring
  float* po = (float*)wlds;  // this wave's output partial [8][128]
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float o0, o1;
      pair32(acc[ct][e], o0, o1);
      if (jr < 2) po[(4 * jr + e) * kHeadDim + 16 * ct + col] = o0 + o1;
    }
  if (lane < 8) {
    part_m[wv][lane] = mref;
    part_l[wv][lane] = lsum;
  }
  __syncthreads();
  for (int idx = tid; idx < hs * kHeadDim; idx += 64 * NW) {
    const int h = idx >> 7, c = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, part_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = part_m[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(part_m[w][h] - M);
      L += f * part_l[w][h];
      O += f * ((const float*)(lds + w * WAVE_LDS))[h * kHeadDim + c];
    }
    const float o = L > 0.f ? O / L : 0.f;
    const float lse = L > 0.f ? (M + __log2f(L)) * kLn2z : -INFINITY;
    if (a.n_splits == 1) {
      const size_t row = (size_t)b * a.n_q_heads + h0 + h;
      a.out[row * kHeadDim + c] = o;
      if (c == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      const size_t row = ((size_t)split * a.batch + b) * a.n_q_heads + h0 + h;
      a.part_o[row * kHeadDim + c] = o;
      if (c == 0) a.part_lse[row] = lse;
    }
  }
}

}  // namespace

hipError_t launch_zip_compress(const ZipCompressArgs& a, int batch, int n_pages, hipStream_t stream) {
  const dim3 grid(n_pages, a.n_kv_heads, batch), block(256);
  hipLaunchKernelGGL(zip_compress_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zip_attention(const ZipAttnArgs& a, int q_type, hipStream_t stream) {
  constexpr int NW = 8, D = 2;
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(64 * NW);
  if (a.heads_per_slice > 8) return hipErrorInvalidValue;
  if (q_type == 0) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 0>), grid, block, 0, stream, a);
  else if (q_type == 1) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 1>), grid, block, 0, stream, a);
  else if (q_type == 2) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 2>), grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq

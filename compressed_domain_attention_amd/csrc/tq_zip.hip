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

template <typename T>
__device__ __forceinline__ T lds_read(const uint8_t* p) {
  return *(const T*)p;
}

// Attention of one (sequence, KV head, section, head slice of up to 8 heads) over its
// tokens, on the matrix unit.  The section's pages go in pairs (32 tokens) to the waves
// in turn; each wave streams its pairs through its own ring of D LDS stages with direct
// global -> LDS copies of exactly the stored bytes (a stage: the pair's key pages, then its
// value pages, each at 4 KB; the metadata of the stage D pairs ahead rides along), so the
// copies in flight cost no registers.
//
// Per pair, with bf16 16x16x32 products:
//   scores S[token][col] = K (16 tokens x 32 coordinates, a key group per lane) x Q (32 x 16)
//     over 4 coordinate blocks, for two 16-token tiles.  Columns are (part, head): the query
//     in BF16 as hi + lo, heads in columns 0-7 (hi) and 8-15 (lo); a lane exchange adds the
//     two parts.  The tiles' rows are chosen so that each lane ends up holding exactly the 8
//     tokens whose value group (8 tokens of one coordinate) the output product pairs it with:
//     tile T row 4j + i is token 8(j&1) + 4T + i of page j>>1.
//   output O[col][coord] += P (16 x 32 tokens) x V (32 x 16 coordinates) for 8 coordinate
//     tiles, the weights as BF16 hi + lo in rows 0-7 and 8-15, straight from the lanes'
//     score registers.
// The softmax reference m is updated lazily (only when a score exceeds it by 8 in log2
// units), so that weights stay in (0, 256]; each wave keeps its own m, sum and output,
// merged across waves at the end.  Results are in the original domain.
template <int NW, int D, int QT>
__global__ __launch_bounds__(64 * NW) void zip_attention_kernel(const ZipAttnArgs a) {
  constexpr int STAGE = 4 * kZipSlot;  // key page A, key page B, value page A, value page B
  constexpr int MSLOT = 256;           // one stage's metadata (32 bytes used)
  constexpr int WAVE_LDS = D * STAGE + 2 * D * MSLOT;
  constexpr int NDMA = 17;             // copies per stage: 4 pages x 4, and the metadata
  static_assert(D >= 2 && D <= 4, "ring depth");
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
  const int npairs = lo < hi ? (pg_hi - pg_lo + 1) >> 1 : 0;  // an empty section (lo = hi = T) has none
  const int n = npairs > wv ? (npairs - wv + NW - 1) / NW : 0;  // this wave's pairs

  const size_t stream = (size_t)b * a.n_kv_heads + kv;
  const uint8_t* ks = a.k_store + stream * a.store_pages * kZipSlot;
  const uint8_t* vs = a.v_store + stream * a.store_pages * kZipSlot;
  const uint8_t* km = a.k_meta + stream * a.store_pages * 8;
  const uint8_t* vm = a.v_meta + stream * a.store_pages * 8;
  const uint8_t* kt = (const uint8_t*)(a.k_tail + stream * a.tail_rows * kHeadDim);
  const uint8_t* vt = (const uint8_t*)(a.v_tail + stream * a.tail_rows * kHeadDim);
  // a start offset is trusted only as far as a whole page slot stays inside the stream
  const uint32_t lim = (uint32_t)max(a.store_pages - 1, 0) * (uint32_t)kZipSlot;

  uint8_t* wlds = lds + wv * WAVE_LDS;                // this wave's ring, then its metadata slots
  uint8_t* mlds = wlds + D * STAGE;
  const uint32_t wlds_a = lds_addr(wlds), mlds_a = lds_addr(mlds);

  auto first_page = [&](int s) { return pg_lo + 2 * (wv + NW * s); };
  // metadata of stage s (its two pages, keys then values) into metadata slot s mod 2D;
  // words of pages outside the store are copied from a valid dummy address
  auto meta_dma = [&](int s) {
    const int p = first_page(s) + ((lane >> 1) & 1);
    const uint8_t* m = (lane & 4) ? vm : km;
    const void* src = (lane < 8 && p < full) ? (const void*)(m + (size_t)p * 8 + 4 * (lane & 1)) : (const void*)kt;
    lds_dma_addr<4, false>(mlds_a + (s % (2 * D)) * MSLOT, src);
  };
  // one 4 KB page region of a stage: `bytes` from `src`; lanes past them copy the first
  // 16 bytes again (into the region's unused part), so every stage issues the same copies
  auto page_dma = [&](uint32_t dst, const uint8_t* src, uint32_t bytes) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t o = 1024u * k + 16u * lane;
      lds_dma_addr<16, true>(dst + 1024u * k, o < bytes ? src + o : src);
    }
  };
  auto page_bytes = [&](uint32_t flags) {
    uint32_t n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) n += ((flags >> (8 * j)) & 0xFFu) == 0xFFu ? 1024u : 768u;
    return n;
  };
  // stage s: the pair's pages (store pages compressed, the open page from the tail buffer,
  // pages past the section not at all), then the metadata of stage s + D
  auto issue = [&](int s) {
    const int p0 = first_page(s);
    const u32x4 mk = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT);
    const u32x4 mv = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT + 16);
    lds_wait();
    const uint32_t dst = wlds_a + (s % D) * STAGE;
#pragma unroll
    for (int P = 0; P < 2; ++P) {
      const int p = p0 + P;
      const uint32_t kst = __builtin_amdgcn_readfirstlane(P ? mk.z : mk.x);
      const uint32_t kfl = __builtin_amdgcn_readfirstlane(P ? mk.w : mk.y);
      const uint32_t vst = __builtin_amdgcn_readfirstlane(P ? mv.z : mv.x);
      const uint32_t vfl = __builtin_amdgcn_readfirstlane(P ? mv.w : mv.y);
      if (p < full) {
        page_dma(dst + P * kZipSlot, ks + min(kst & ~15u, lim), page_bytes(kfl));
        page_dma(dst + (2 + P) * kZipSlot, vs + min(vst & ~15u, lim), page_bytes(vfl));
      } else if (p < pg_hi) {
        const size_t row = (size_t)((16 * p) % a.tail_rows) * 256;
        page_dma(dst + P * kZipSlot, kt + row, kZipSlot);
        page_dma(dst + (2 + P) * kZipSlot, vt + row, kZipSlot);
      } else {
        page_dma(dst + P * kZipSlot, kt, 0);
        page_dma(dst + (2 + P) * kZipSlot, vt, 0);
      }
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
  const int jr = lane >> 4;  // row group: score rows 4 jr .. 4 jr + 3, operand k = 8 jr ..

  for (int s = 0; s < n; ++s) {
    const int younger = min(D - 1, n - 1 - s);
    if (younger >= 3) vm_wait<3 * NDMA>();
    else if (younger == 2) vm_wait<2 * NDMA>();
    else if (younger == 1) vm_wait<NDMA>();
    else vm_wait<0>();
    const int p0 = first_page(s);
    const u32x4 mk = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT);
    const u32x4 mv = lds_read<u32x4>(mlds + (s % (2 * D)) * MSLOT + 16);
    const uint8_t* sb = wlds + (s % D) * STAGE;
    const int nA = min(16, hi - 16 * p0), nB = p0 + 1 < pg_hi ? min(16, hi - 16 * (p0 + 1)) : 0;
    // page kinds: 0 stored, 1 open (BF16 tail rows), 2 absent
    const int kA = p0 < full ? 0 : 1, kB = p0 + 1 < full ? 0 : (p0 + 1 < pg_hi ? 1 : 2);

    // ---- scores: two 16-token tiles
    f32x4 sc[2];
    {
      const int r = col, j = r >> 2, i = r & 3, P = j >> 1;
      const int kind = P ? kB : kA;
      const uint32_t flags = kind == 0 ? (P ? mk.w : mk.y) : kKept;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        uint32_t off, mode;
        chunk_at(flags, 2 * (j & 1) + t, off, mode);
        const uint8_t* cb = sb + P * kZipSlot + off;
        f32x4 acc_s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int g = 4 * kb + jr;  // group of the token: coordinates 8g .. 8g + 7
          u32x4 kop;
          if (mode == kKept) kop = lds_read<u32x4>(cb + 256 * i + 16 * g);
          else kop = decode_group(lds_read<u32x2>(cb + 128 * i + 8 * g), lds_read<uint32_t>(cb + 512 + 64 * i + 4 * g), mode);
          acc_s = mfma_bf16(kop, qf[kb], acc_s);
        }
        sc[t] = acc_s;
      }
    }
    // hi + lo parts, scale, mask; this lane's rows: tile t row 4 jr + e = token
    // 8 (jr & 1) + 4 t + e of page jr >> 1
    float x[2][4];
    float bm = -INFINITY;
    {
      const int np = (jr >> 1) ? nB : nA;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = (sc[t][e] + dpp<0x128>(sc[t][e])) * a.scale_log2;
          x[t][e] = 8 * (jr & 1) + 4 * t + e < np ? v : -INFINITY;
          bm = fmaxf(bm, x[t][e]);
        }
    }
    bm = fmaxf(bm, lane_xor(bm, 16, lane));
    bm = fmaxf(bm, lane_xor(bm, 32, lane));
    if (__builtin_amdgcn_ballot_w64(bm > thr)) {
      const float mnew = fmaxf(mref, bm);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);  // 0 on the first block
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
    // weights: BF16 hi (columns 0-7) or lo (8-15) parts, in the operand's k order
    u32x4 pf;
    {
      float p[2][4];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[t][e] = __builtin_amdgcn_exp2f(x[t][e] - mref);
          lsum += p[t][e];
          if (col >= 8) p[t][e] = bf16_lo(p[t][e]);
        }
      pf = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                 pack_bf16(p[1][2], p[1][3])};
    }

    // ---- output: 8 coordinate tiles; lane holds coordinate 16 ct + col, tokens
    // 8 (jr & 1) .. + 7 of page jr >> 1 (a value group)
    {
      const int P = jr >> 1, hh = jr & 1;
      const int kind = P ? kB : kA;
      const int np = P ? nB : nA;
      const uint32_t flags = P ? mv.w : mv.y;
      const uint8_t* pb = sb + (2 + P) * kZipSlot;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int d = 16 * ct + col;
        u32x4 vop;
        if (kind == 0) {
          uint32_t off, mode;
          chunk_at(flags, ct >> 1, off, mode);
          const int g = 2 * (d & 31) + hh;
          if (mode == kKept) vop = lds_read<u32x4>(pb + off + 16 * g);
          else vop = decode_group(lds_read<u32x2>(pb + off + 8 * g), lds_read<uint32_t>(pb + off + 512 + 4 * g), mode);
        } else if (kind == 1) {
          // the open page, token-major BF16: gather the group, zero tokens past the row
          uint32_t w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int t = 8 * hh + e;
            w[e] = t < np ? (uint32_t)lds_read<uint16_t>(pb + 256 * t + 2 * d) : 0u;
          }
          vop = u32x4{w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16), w[6] | (w[7] << 16)};
        } else {
          vop = u32x4{0u, 0u, 0u, 0u};
        }
        acc[ct] = mfma_bf16(pf, vop, acc[ct]);
      }
    }
    // the stage's slot is refilled with stage s + D once its reads are done
    if (s + D < n) {
      lds_wait();
      issue(s + D);
    }
  }

  // ---- merge the waves: sums over the row groups, hi + lo output rows
  vm_wait<0>();
  lsum += lane_xor(lsum, 16, lane);
  lsum += lane_xor(lsum, 32, lane);
  __syncthreads();  // every wave is done with its ring
  float* po = (float*)wlds;  // this wave's output partial [8][128]
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float o = acc[ct][e] + lane_xor(acc[ct][e], 32, lane);
      if (jr < 2) po[(4 * jr + e) * kHeadDim + 16 * ct + col] = o;
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
  constexpr int NW = 4, D = 2;
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(64 * NW);
  if (a.heads_per_slice > 8) return hipErrorInvalidValue;
  if (q_type == 0) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 0>), grid, block, 0, stream, a);
  else if (q_type == 1) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 1>), grid, block, 0, stream, a);
  else if (q_type == 2) hipLaunchKernelGGL((zip_attention_kernel<NW, D, 2>), grid, block, 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tq

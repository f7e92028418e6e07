// HIP kernels of the lossless BF16 exponent codec of a KV cache and of decode attention
// read straight from the compressed pages.  Target: gfx950 (MI355X), wave64.
//
// Method source: "ZipFusion: Fusing Lossless KV Decompression with Attention for Efficient
// LLM Decoding" (paper-daily.com): the compression format (only the exponent is coded: a
// chunk of 512 values keeps every low byte and replaces the rest by a 4-bit sign + exponent
// offset code against the chunk's even base b, when all exponents lie in [b, b + 15]), the
// page layout (16-token pages, 4 key and 4 value chunks per page and head, 8 bytes of
// metadata each) and the register decode (the high byte of a value is sign * 128 + b/2 + d:
// one 32-bit add of b/2 in every byte yields four high bytes, with no rounding).
//
// Layout of one (sequence, KV head) stream, for keys and for values alike:
//   store [page][4096 bytes]: the page's 4 chunks back to back from the slot start, each
//     either compressed (512 low bytes, then 256 code bytes) or kept (1024 bytes of BF16);
//     the rest of the slot is zero.  Chunk c of a page holds its tokens 4c .. 4c + 3.
//   meta [page][8 bytes]: little-endian u32 byte offset of the page's first chunk in the
//     stream, then one byte per chunk: 0xFF for a kept chunk, else b/2.
//   Code byte 4g + j of a chunk holds value 8g + j (sign bit 7, d bits 0-2) and value
//     8g + j + 4 (sign bit 6, d bits 3-5), d = (exponent - b) / 2 rounded down.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tq_internal.h"
#include "tq_lanes.h"

namespace tq {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2z = 0.69314718055994531f;
constexpr uint32_t kKept = 0xFFFFFFFFu;  // decode mode of a kept (uncompressed) chunk

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
// Compression of whole pages.  One workgroup per (page, KV head, sequence); wave c codes
// chunk c; lane l holds the chunk's values 8l .. 8l + 7 (one 16-byte load), i.e. the eight
// values that share four code bytes.
__global__ __launch_bounds__(256) void zip_compress_kernel(const ZipCompressArgs a) {
  __shared__ uint32_t flag[4];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, c = tid >> 6;
  const size_t stream = (size_t)b * a.n_kv_heads + h;
  const uint16_t* src =
      a.x + (stream * a.x_rows + (size_t)kZipPage * (a.src_page0 + i)) * kHeadDim + 512 * c + 8 * lane;
  const uint4 w = *(const uint4*)src;
  const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
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
    // low bytes of the 8 values (bytes 0 and 2 of each 32-bit word)
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
    *(uint4*)(dst + off + 16 * lane) = w;
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
// Register decode of eight coded values (one code word): the high bytes of values 1-4 are
// the code word masked with 0x87878787 plus b/2 in every byte, those of values 5-8 the code
// word shifted into the same places; a byte permute then joins each high byte with its low
// byte under 16 zero bits, which is the value as an fp32.
__device__ __forceinline__ void decode8(uint32_t lo0, uint32_t lo1, uint32_t code, uint32_t bh4, float* out) {
  const uint32_t h1 = (code & 0x87878787u) + bh4;
  const uint32_t h5 = (((code >> 3) & 0x07070707u) | ((code << 1) & 0x80808080u)) + bh4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t sel = ((uint32_t)(4 + j) << 24) | ((uint32_t)j << 16) | 0x0C0Cu;
    out[j] = __uint_as_float(__builtin_amdgcn_perm(h1, lo0, sel));
    out[j + 4] = __uint_as_float(__builtin_amdgcn_perm(h5, lo1, sel));
  }
}

// Eight BF16 values kept as they are (four 32-bit words) as fp32.
__device__ __forceinline__ void widen8(uint4 w, float* out) {
  const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(x[j] << 16);
    out[2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u);
  }
}

// Where token row t4 of chunk c of a page lies: the chunk's byte offset from the page start
// and its decode mode (kKept, or b/2 in every byte).
__device__ __forceinline__ void chunk_at(uint32_t flags, int c, uint32_t& off, uint32_t& mode) {
  off = 768u * (uint32_t)c;
#pragma unroll
  for (int j = 0; j < 3; ++j) off += (j < c && ((flags >> (8 * j)) & 0xFFu) == 0xFFu) ? 256u : 0u;
  const uint32_t f = (flags >> (8 * c)) & 0xFFu;
  mode = f == 0xFFu ? kKept : (f & 0x7Fu) * 0x01010101u;
}

// Attention of one (sequence, KV head, section, head slice) over its tokens.  Full pages are
// read compressed and decoded in registers; tokens past the last full page come from the
// BF16 tail buffer.  64-token chunks as four whole pages: thread (token, quarter) forms
// 32-coordinate partial scores for every head, summed over the quarter lanes; one wave per
// head runs the online softmax over the chunk; thread (8 coordinates, token slot) adds 4
// tokens of the chunk, one per page, for every head.  Results stay in the original domain.
template <int MAXH, int QT>
__global__ __launch_bounds__(256) void zip_attention_kernel(const ZipAttnArgs a) {
  __shared__ __attribute__((aligned(16))) float qb[MAXH * kHeadDim];  // scaled query, later the output
  __shared__ float pw[MAXH][64];                                      // chunk scores, then weights
  __shared__ float hm[MAXH], hsum[MAXH], halpha[MAXH];
  __shared__ __attribute__((aligned(16))) float ob[4][MAXH][kHeadDim];  // per-wave value sums
  __shared__ float lse2[MAXH];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int unit = blockIdx.x / a.n_slices, slice = blockIdx.x - unit * a.n_slices;
  const int split = unit % a.n_splits, kv = (unit / a.n_splits) % a.n_kv_heads;
  const int b = unit / (a.n_splits * a.n_kv_heads);
  const int h0 = kv * a.group_size + slice * a.heads_per_slice;
  const int hs = min(a.heads_per_slice, a.group_size - slice * a.heads_per_slice);
  // lengths beyond max_len (checked against the store and the tail on the host) are clamped
  const int T = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_len)) : a.max_len;
  const int full = min(T >> 4, a.store_pages);  // pages read from the store
  // sections of whole pages, so that every 64-token chunk is four pages
  const int C = (((T + a.n_splits - 1) / a.n_splits) + 15) & ~15;
  const int lo = min(T, split * C), hi = min(T, lo + C);

  const size_t stream = (size_t)b * a.n_kv_heads + kv;
  const uint8_t* ks = a.k_store + stream * a.store_pages * kZipSlot;
  const uint8_t* vs = a.v_store + stream * a.store_pages * kZipSlot;
  const uint8_t* kmeta = a.k_meta + stream * a.store_pages * 8;
  const uint8_t* vmeta = a.v_meta + stream * a.store_pages * 8;
  const uint8_t* kt = (const uint8_t*)(a.k_tail + stream * a.tail_rows * kHeadDim);
  const uint8_t* vt = (const uint8_t*)(a.v_tail + stream * a.tail_rows * kHeadDim);
  // a start offset is trusted only as far as a whole page slot stays inside the stream
  const uint32_t lim = (uint32_t)max(a.store_pages - 1, 0) * (uint32_t)kZipSlot;

  const int st = tid >> 2, qd = tid & 3;   // scores: token, quarter
  const int dg = tid & 15, ts = tid >> 4;  // values: 8 coordinates, token slot within a page

  // (start, flags) of a page's metadata; pages past the stored ones are never read
  auto page_meta = [&](const uint8_t* meta, int p) {
    return p < full ? *(const u32x2*)(meta + (size_t)p * 8) : u32x2{0u, 0xFFFFFFFFu};
  };
  // the score token's 32 key values (this wave's page of the chunk): coded, two words of
  // low bytes and one of codes; kept or tail, four words of BF16 pairs
  auto fetch_k = [&](int c0, u32x2 m, uint4& w0, uint4& w1, uint4& w2, uint4& w3, uint32_t& mode) {
    const int tk = c0 + st;
    if (tk >= hi) return;  // past the section: not read, masked
    const uint8_t* a0;
    const uint8_t* a2;
    uint32_t md = kKept;
    if ((tk >> 4) < full) {
      uint32_t off;
      chunk_at(m.y, (st >> 2) & 3, off, md);
      const uint8_t* cb = ks + min(m.x & ~15u, lim) + off;
      const int t4 = st & 3;
      a0 = md == kKept ? cb + 256 * t4 + 64 * qd : cb + 128 * t4 + 32 * qd;
      a2 = md == kKept ? a0 + 32 : cb + 512 + 64 * t4 + 16 * qd;
    } else {
      a0 = kt + (size_t)(tk % a.tail_rows) * 256 + 64 * qd;
      a2 = a0 + 32;
    }
    w0 = *(const uint4*)a0;
    w1 = *(const uint4*)(a0 + 16);
    w2 = *(const uint4*)a2;
    if (md == kKept) w3 = *(const uint4*)(a2 + 16);
    mode = md;
  };
  // token ts of page j of the chunk, coordinates 8dg .. +7: coded, x and y the low bytes and
  // z the code word; kept or tail, four words of BF16 pairs
  auto fetch_v = [&](int c0, int j, u32x2 m, uint4& w, uint32_t& mode) {
    const int tv = c0 + 16 * j + ts;
    if (tv >= hi) return;
    if ((tv >> 4) < full) {
      uint32_t off, md;
      chunk_at(m.y, ts >> 2, off, md);
      const uint8_t* cb = vs + min(m.x & ~15u, lim) + off;
      const int t4 = ts & 3;
      if (md == kKept) {
        w = *(const uint4*)(cb + 256 * t4 + 16 * dg);
      } else {
        const u32x2 l = *(const u32x2*)(cb + 128 * t4 + 8 * dg);
        w = make_uint4(l.x, l.y, *(const uint32_t*)(cb + 512 + 64 * t4 + 4 * dg), 0u);
      }
      mode = md;
    } else {
      w = *(const uint4*)(vt + (size_t)(tv % a.tail_rows) * 256 + 16 * dg);
      mode = kKept;
    }
  };

  // the next chunk's raw words and the metadata of the chunk after it
  uint4 nk0, nk1, nk2, nk3, nv0, nv1, nv2, nv3;
  uint32_t nkm = kKept, nvm0 = kKept, nvm1 = kKept, nvm2 = kKept, nvm3 = kKept;
  u32x2 mk, mv0, mv1, mv2, mv3;
  auto load_meta = [&](int c0) {
    const int p0 = c0 >> 4;
    mk = page_meta(kmeta, p0 + wv);
    mv0 = page_meta(vmeta, p0);
    mv1 = page_meta(vmeta, p0 + 1);
    mv2 = page_meta(vmeta, p0 + 2);
    mv3 = page_meta(vmeta, p0 + 3);
  };
  auto fetch = [&](int c0) {
    fetch_k(c0, mk, nk0, nk1, nk2, nk3, nkm);
    fetch_v(c0, 0, mv0, nv0, nvm0);
    fetch_v(c0, 1, mv1, nv1, nvm1);
    fetch_v(c0, 2, mv2, nv2, nvm2);
    fetch_v(c0, 3, mv3, nv3, nvm3);
  };
  if (lo < hi) {
    load_meta(lo);
    fetch(lo);  // the first chunk's reads overlap the query set-up
    if (lo + 64 < hi) load_meta(lo + 64);
  }

  for (int i = tid; i < hs * kHeadDim; i += 256) {
    const size_t qi = ((size_t)b * a.n_q_heads + h0 + (i >> 7)) * kHeadDim + (i & 127);
    float x;
    if (QT == 1) x = (float)((const _Float16*)a.q)[qi];
    else if (QT == 2) x = __uint_as_float((uint32_t)((const uint16_t*)a.q)[qi] << 16);
    else x = ((const float*)a.q)[qi];
    qb[i] = x * a.scale_log2;
  }
  if (tid < MAXH) {
    hm[tid] = -INFINITY;
    hsum[tid] = 0.f;
  }
  __syncthreads();

  float acc[MAXH][8];
#pragma unroll
  for (int h = 0; h < MAXH; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  for (int c0 = lo; c0 < hi; c0 += 64) {
    const uint4 k0 = nk0, k1 = nk1, k2 = nk2, k3 = nk3;
    const uint4 cv[4] = {nv0, nv1, nv2, nv3};
    const uint32_t km = nkm, vmode[4] = {nvm0, nvm1, nvm2, nvm3};
    if (c0 + 64 < hi) {
      fetch(c0 + 64);  // the next chunk loads during this one
      if (c0 + 128 < hi) load_meta(c0 + 128);
    }
    // scores of the chunk's tokens, all heads (scale and log2 e folded into the query)
    {
      const int tok = c0 + st;
      float kx[32];
      if (km == kKept) {
        widen8(k0, kx);
        widen8(k1, kx + 8);
        widen8(k2, kx + 16);
        widen8(k3, kx + 24);
      } else {
        decode8(k0.x, k0.y, k2.x, km, kx);
        decode8(k0.z, k0.w, k2.y, km, kx + 8);
        decode8(k1.x, k1.y, k2.z, km, kx + 16);
        decode8(k1.z, k1.w, k2.w, km, kx + 24);
      }
#pragma unroll
      for (int h = 0; h < MAXH; ++h) {
        if (h < hs) {
          const float4* qp = (const float4*)(qb + h * kHeadDim + 32 * qd);
          float sc = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float4 qq = qp[i];
            sc = fmaf(qq.x, kx[4 * i], sc);
            sc = fmaf(qq.y, kx[4 * i + 1], sc);
            sc = fmaf(qq.z, kx[4 * i + 2], sc);
            sc = fmaf(qq.w, kx[4 * i + 3], sc);
          }
          sc += lane_xor(sc, 1, lane);
          sc += lane_xor(sc, 2, lane);
          if (qd == 0) pw[h][st] = tok < hi ? sc : -INFINITY;  // tokens past the section are masked
        }
      }
    }
    __syncthreads();
    // online softmax per head over the chunk (log2 units)
    for (int h = wv; h < hs; h += 4) {
      const float sc = pw[h][lane];
      float bm = sc;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) bm = fmaxf(bm, lane_xor(bm, o, lane));
      const float mold = hm[h];
      const float mnew = fmaxf(mold, bm);
      const float al = mnew > mold ? __builtin_amdgcn_exp2f(mold - mnew) : 1.f;
      const float mu = mnew == -INFINITY ? 0.f : mnew;
      const float p = __builtin_amdgcn_exp2f(sc - mu);
      float psum = p;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) psum += lane_xor(psum, o, lane);
      pw[h][lane] = p;
      if (lane == 0) {
        hm[h] = mnew;
        hsum[h] = hsum[h] * al + psum;
        halpha[h] = al;
      }
    }
    __syncthreads();
    // value sums: token ts of each of the chunk's four pages, coordinates 8dg .. +7
    {
#pragma unroll
      for (int h = 0; h < MAXH; ++h) {
        if (h < hs) {
          const float al = halpha[h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + 16 * j + ts < hi) {
          float vx[8];
          if (vmode[j] == kKept) widen8(cv[j], vx);
          else decode8(cv[j].x, cv[j].y, cv[j].z, vmode[j], vx);
#pragma unroll
          for (int h = 0; h < MAXH; ++h) {
            if (h < hs) {
              const float p = pw[h][16 * j + ts];
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vx[e], acc[h][e]);
            }
          }
        }
      }
    }
    __syncthreads();  // the weights are rewritten by the next chunk
  }

  // sum the 16 token slots (lane bits 4, 5, then the four waves), normalise
#pragma unroll
  for (int h = 0; h < MAXH; ++h) {
    if (h < hs) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = acc[h][e];
        x += lane_xor(x, 16, lane);
        x += lane_xor(x, 32, lane);
        if ((lane >> 4) == 0) ob[wv][h][8 * dg + e] = x;
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < hs * kHeadDim; i += 256) {
    const int h = i >> 7, c = i & 127;
    const float L = hsum[h];
    qb[i] = L > 0.f ? (ob[0][h][c] + ob[1][h][c] + ob[2][h][c] + ob[3][h][c]) / L : 0.f;
    if (c == 0) lse2[h] = L > 0.f ? hm[h] + __log2f(L) : -INFINITY;
  }
  __syncthreads();
  if (a.n_splits == 1) {
    const size_t row = (size_t)b * a.n_q_heads + h0;
    if (a.lse_out && tid < hs) a.lse_out[row + tid] = lse2[tid] * kLn2z;
    for (int i = tid; i < hs * kHeadDim; i += 256) a.out[(row + (i >> 7)) * kHeadDim + (i & 127)] = qb[i];
  } else {
    const size_t prow = ((size_t)split * a.batch + b) * a.n_q_heads + h0;
    if (tid < hs) a.part_lse[prow + tid] = lse2[tid] * kLn2z;
    for (int i = tid; i < hs * kHeadDim; i += 256) a.part_o[(prow + (i >> 7)) * kHeadDim + (i & 127)] = qb[i];
  }
}

}  // namespace

hipError_t launch_zip_compress(const ZipCompressArgs& a, int batch, int n_pages, hipStream_t stream) {
  const dim3 grid(n_pages, a.n_kv_heads, batch), block(256);
  hipLaunchKernelGGL(zip_compress_kernel, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_zip_attention(const ZipAttnArgs& a, int q_type, hipStream_t stream) {
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(256);
#define TQ_ZIP(H, Q)                                                                 \
  if (a.heads_per_slice <= H && q_type == Q) {                                       \
    hipLaunchKernelGGL((zip_attention_kernel<H, Q>), grid, block, 0, stream, a);     \
    return hipGetLastError();                                                        \
  }
#define TQ_ZIP_Q(H) TQ_ZIP(H, 0) TQ_ZIP(H, 1) TQ_ZIP(H, 2)
  TQ_ZIP_Q(4) TQ_ZIP_Q(8)
#undef TQ_ZIP_Q
#undef TQ_ZIP
  return hipErrorInvalidValue;
}

}  // namespace tq

// HIP kernels for decode attention on a rotated, Lloyd-Max-quantised, bit-packed KV cache.
// Target: gfx950 (MI355X), wave64.
//
// Method sources (page, section): "TurboQuant: ... MNN on phones" 2.1-2.3 and 3.1-3.4
// (norm -> rotate -> per-coordinate codebook search; block-32 Walsh-Hadamard with sign
// flips; rotated-domain key dot and value sum); "RotaryQuant ... Fused Compressed-Space
// Attention", key designs 2-3 (Hadamard followed by SO(4) block rotations; rotate the
// query once and the output once); "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", packed-cache implementation details (key-axis split, log-sum-exp merge,
// whole-prompt quantisation in one call).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994531f;

// Position of tile token t inside a tile's norm block (layout in tq.h).
__device__ __forceinline__ int norm_pos(int t) { return 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3); }

__device__ __forceinline__ uint32_t f16_bits(_Float16 h) { return (uint32_t)__builtin_bit_cast(uint16_t, h); }

// Forward rotation of up to eight query heads in registers: wave w, lane l holds head
// 2w + (l >> 5), coordinates 4(l & 31) .. +3 (one SO(4) block).  The first two Hadamard
// stages are in-lane, the rest exchange with lane l ^ m inside the 32-lane half.  The
// global reads are issued by query_fetch, early, so that their latency overlaps the
// decode-table setup; query_rotate does the arithmetic.
struct QueryLane {
  float4 x, sg;
  Quat l, r;
  bool live;
};

template <bool QF16>
__device__ __forceinline__ QueryLane query_fetch(const float* signs, const float* so4, const void* q,
                                                 size_t row0, int hs, int wv, int lane) {
  QueryLane s;
  const int hl = 2 * wv + (lane >> 5), p = lane & 31;
  s.live = hl < hs;
  s.x = make_float4(0.f, 0.f, 0.f, 0.f);
  s.sg = s.x;
  s.l = s.r = Quat{1.f, 0.f, 0.f, 0.f};
  if (s.live) {
    const size_t qi = (row0 + hl) * kHeadDim + 4 * p;
    if (QF16) {
      typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
      const h4_t h = *(const h4_t*)((const _Float16*)q + qi);
      s.x = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
    } else {
      s.x = *(const float4*)((const float*)q + qi);
    }
    s.sg = *(const float4*)(signs + 4 * p);
    if (so4) {
      s.l = qload(so4 + 8 * p);
      s.r = qload(so4 + 8 * p + 4);
    }
  }
  return s;
}

// The same lane values read back from LDS, where direct copies staged them: the raw
// query rows of this wave's two heads at qraw (fp32 rows of 128, or fp16 rows packed), the
// signs and then the SO(4) parameters at stage.
template <bool QF16>
__device__ __forceinline__ QueryLane query_staged(const uint8_t* qraw, const float* stage, bool so4, int hs, int wv,
                                                 int lane) {
  QueryLane s;
  const int hl = 2 * wv + (lane >> 5), p = lane & 31;
  s.live = hl < hs;
  s.x = make_float4(0.f, 0.f, 0.f, 0.f);
  s.sg = s.x;
  s.l = s.r = Quat{1.f, 0.f, 0.f, 0.f};
  if (s.live) {
    const int i = (lane >> 5) * kHeadDim + 4 * p;
    if (QF16) {
      typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
      const h4_t h = *(const h4_t*)(qraw + 2 * i);
      s.x = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
    } else {
      s.x = *(const float4*)(qraw + 4 * i);
    }
    s.sg = *(const float4*)(stage + 4 * p);
    if (so4) {
      s.l = qload(stage + kHeadDim + 8 * p);
      s.r = qload(stage + kHeadDim + 8 * p + 4);
    }
  }
  return s;
}

template <int GROUP>
__device__ __forceinline__ float4 query_rotate(const QueryLane& s, bool so4, int lane) {
  constexpr int group = GROUP;
  float x0 = s.x.x * s.sg.x, x1 = s.x.y * s.sg.y, x2 = s.x.z * s.sg.z, x3 = s.x.w * s.sg.w;
  float y0 = x0 + x1, y1 = x0 - x1, y2 = x2 + x3, y3 = x2 - x3;
  x0 = y0 + y2; x1 = y1 + y3; x2 = y0 - y2; x3 = y1 - y3;
#pragma unroll
  for (int m = 1; m < group / 4; m <<= 1) {
    const bool up = (lane & m) != 0;
    const float o0 = lane_xor(x0, m, lane), o1 = lane_xor(x1, m, lane), o2 = lane_xor(x2, m, lane),
                o3 = lane_xor(x3, m, lane);
    x0 = up ? o0 - x0 : x0 + o0;
    x1 = up ? o1 - x1 : x1 + o1;
    x2 = up ? o2 - x2 : x2 + o2;
    x3 = up ? o3 - x3 : x3 + o3;
  }
  const float hsc = group == 32 ? 0.17677669529663688f : 0.088388347648318440f;
  Quat v{x0 * hsc, x1 * hsc, x2 * hsc, x3 * hsc};
  if (so4) v = qmul(qmul(s.l, v), qconj(s.r));
  return make_float4(v.w, v.x, v.y, v.z);
}

// Bit field of width W at bit offset `off` of a little-endian dword array; `off` and W
// are compile-time constants after unrolling.
template <int W>
__device__ __forceinline__ uint32_t field(const uint32_t* d, int off) {
  const int wi = off >> 5, sh = off & 31;
  const uint32_t x = (sh + W <= 32) ? (d[wi] >> sh) : __builtin_amdgcn_alignbit(d[wi + 1], d[wi], sh);
  return x & ((1u << W) - 1u);
}

// ---------------------------------------------------------------------------------------
// Append: fused norm + sign flip + Walsh-Hadamard + [SO(4)] + codebook search + pack.
// One workgroup of 128 threads owns one 32-slot tile of one (sequence, KV head); thread
// (token, chunk) holds 32 consecutive coordinates in registers.  The 32-point transform
// runs in registers; a whole-head (128) transform adds two cross-lane stages.
template <int BITS, int GROUP, bool VALUES, bool XF16>
__device__ __forceinline__ void append_tile(const AppendArgs& a, int b, int h, int tile) {
  constexpr int NB = (1 << BITS) - 1;
  constexpr int NG = kHeadDim / GROUP;
  constexpr int ND = BITS;  // dwords of the four value words a thread merges
  __shared__ uint32_t tile_codes[VALUES ? kTile * kHeadDim / 4 : 1];  // u8 [32][128]
  const int tid = threadIdx.x, tok = tid >> 2, chunk = tid & 3;
  const int pos = a.pos ? a.pos[b] : a.pos0;
  const int t0 = (pos / kTile + tile) * kTile;
  if (t0 >= pos + a.n_new) return;  // uniform over the block
  const int slot = t0 + tok;
  const bool valid = slot >= pos && slot < pos + a.n_new;
  const size_t stream = (size_t)b * a.n_kv_heads + h;
  const int ntile = a.capacity / kTile;

  // Reads that do not depend on the new vectors are issued first, beside the vector load:
  // the SO(4) parameters of this thread's eight 4-blocks, and the packed value words this
  // thread merges when the tile is only partly rewritten.
  Quat ql[8], qr[8];
  if (a.so4 != nullptr) {
    const float* qp = a.so4 + ((size_t)h * 32 + chunk * 8) * 8;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ql[k] = qload(qp + 8 * k);
      qr[k] = qload(qp + 8 * k + 4);
    }
  }
  const int vlo = pos > t0 ? pos - t0 : 0;
  const int vhi = min(kTile, pos + a.n_new - t0);
  const bool partial = vlo > 0 || vhi < kTile;
  uint32_t* vo = VALUES ? (uint32_t*)(a.codes + (stream * ntile + t0 / kTile) * (kTile * 16 * BITS) + 4 * tid * BITS)
                        : nullptr;
  uint32_t old[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) old[j] = 0u;
  if (VALUES && partial) {
#pragma unroll
    for (int j = 0; j < ND; ++j) old[j] = vo[j];
  }

  float v[32];
  if (valid) {
    const size_t row = (stream * a.n_new + (slot - pos)) * kHeadDim + chunk * 32;
    if (XF16) {
      const uint4* p = (const uint4*)((const _Float16*)a.x + row);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t hv = __builtin_bit_cast(half8_t, p[j]);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * j + e] = (float)hv[e];
      }
    } else {
      const float4* p = (const float4*)((const float*)a.x + row);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float4 f = p[j];
        v[4 * j] = f.x; v[4 * j + 1] = f.y; v[4 * j + 2] = f.z; v[4 * j + 3] = f.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
  }

  // sign flips (exact) and the group's squared norm
  const float4* sp = (const float4*)(a.signs + h * kHeadDim + chunk * 32);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float4 s = sp[j];
    v[4 * j] *= s.x; v[4 * j + 1] *= s.y; v[4 * j + 2] *= s.z; v[4 * j + 3] *= s.w;
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) ss = fmaf(v[i], v[i], ss);
  if (GROUP == 128) {
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
  }
  const float nrm = sqrtf(ss);
  const float inv = nrm > 0.f ? 1.0f / nrm : 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= inv;

  // 32-point Walsh-Hadamard butterfly in registers (Sylvester order)
#pragma unroll
  for (int s = 1; s < 32; s <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & s) == 0) {
        const float x0 = v[i], x1 = v[i + s];
        v[i] = x0 + x1;
        v[i + s] = x0 - x1;
      }
    }
  }
  if (GROUP == 128) {  // coordinate bits 5 and 6 live in the lane's chunk index
#pragma unroll
    for (int st = 1; st <= 2; st <<= 1) {
      const bool upper = (chunk & st) != 0;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float o = __shfl_xor(v[i], st);
        v[i] = upper ? (o - v[i]) : (v[i] + o);
      }
    }
  }
  const float hs = GROUP == 32 ? 0.17677669529663688f : 0.088388347648318440f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] *= hs;

  if (a.so4 != nullptr) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const Quat o = qmul(qmul(ql[k], Quat{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]}), qconj(qr[k]));
      v[4 * k] = o.w; v[4 * k + 1] = o.x; v[4 * k + 2] = o.y; v[4 * k + 3] = o.z;
    }
  }

  // code = number of boundaries strictly below the value
  uint32_t code[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < NB; ++k) c += v[i] > a.boundary[k] ? 1u : 0u;
    code[i] = c;
  }

  if (valid && (GROUP == 32 || chunk == 0)) {
    const int grp = GROUP == 32 ? chunk : 0;
    a.norms[(stream * ntile + t0 / kTile) * (NG * kTile) + grp * kTile + norm_pos(tok)] = nrm;
  }

  if (!VALUES) {
    if (valid) {
      uint32_t* o = (uint32_t*)(a.codes + (stream * a.capacity + slot) * (16 * BITS) + chunk * (4 * BITS));
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t x = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) x |= code[8 * j + e] << (BITS * e);
        w[j] = x;
      }
      if (BITS == 3) {
        o[0] = w[0] | (w[1] << 24);
        o[1] = (w[1] >> 8) | (w[2] << 16);
        o[2] = (w[2] >> 16) | (w[3] << 8);
      } else {
        *(uint4*)o = make_uint4(w[0], w[1], w[2], w[3]);
      }
    }
    return;
  }

  // values: stage byte codes of the whole tile, then emit 8-token words
  uint8_t* tc = (uint8_t*)tile_codes;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    tile_codes[(tok * kHeadDim + chunk * 32) / 4 + j] =
        code[4 * j] | (code[4 * j + 1] << 8) | (code[4 * j + 2] << 16) | (code[4 * j + 3] << 24);
  }
  __syncthreads();
  const int w0 = 4 * tid;  // four consecutive words: same (q, m), u = u0..u0+3
  const int q = w0 >> 7, m = (w0 >> 3) & 15, u0 = w0 & 7;
  uint32_t word[4], mask[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 16 * (u0 + j) + m;
    uint32_t x = 0, mk = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int t = 16 * (k >> 2) + 4 * q + (k & 3);
      if (t >= vlo && t < vhi) {
        x |= (uint32_t)tc[t * kHeadDim + i] << (BITS * k);
        mk |= (uint32_t)NB << (BITS * k);
      }
    }
    word[j] = x;
    mask[j] = mk;
  }
  uint32_t dv[4], dm[4];
  if (BITS == 3) {
    dv[0] = word[0] | (word[1] << 24); dv[1] = (word[1] >> 8) | (word[2] << 16); dv[2] = (word[2] >> 16) | (word[3] << 8);
    dm[0] = mask[0] | (mask[1] << 24); dm[1] = (mask[1] >> 8) | (mask[2] << 16); dm[2] = (mask[2] >> 16) | (mask[3] << 8);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) { dv[j] = word[j]; dm[j] = mask[j]; }
  }
#pragma unroll
  for (int j = 0; j < ND; ++j) {
    if (dm[j] == 0xFFFFFFFFu) vo[j] = dv[j];
    else if (dm[j] != 0u) vo[j] = (old[j] & ~dm[j]) | dv[j];
  }
}

template <int BITS, int GROUP, bool VALUES, bool XF16>
__global__ __launch_bounds__(128) void append_kernel(const AppendArgs a) {
  append_tile<BITS, GROUP, VALUES, XF16>(a, blockIdx.z, blockIdx.y, a.n_edges ? a.edge[blockIdx.x] : blockIdx.x);
}

// One new token per (sequence, KV head), keys and values together: one wave per stream,
// lanes 0-31 quantise the key and lanes 32-63 the value, lane l & 31 holding coordinates
// 4(l & 31) .. +3 (one SO(4) block).  Same steps as append_tile (norm, signs, normalised
// Hadamard with the first two stages in-lane and the rest by lane exchange, SO(4), count
// of boundaries below, pack); the group norm is summed in another order, so results may
// differ from append_tile in the last bit of a norm.  Value codes are merged byte by byte:
// every byte a lane writes belongs to its own words.
// One wave appends the token of stream st = b * n_kv_heads + kv; x_f16 selects the vector
// type.  Shared by the append kernel below and by the decode kernel's fused append.
template <int BK, int BV, int GROUP>
__device__ __forceinline__ void append_step_wave(const AppendArgs& ak, const AppendArgs& av, int st, bool x_f16,
                                                 int lane) {
  constexpr int NG = kHeadDim / GROUP;
  const bool val = lane >= 32;
  // the lane's own cache, field by field (a lane-selected reference to either argument
  // block would be copied to private memory); positions, signs and SO(4) are common
  const int bits = val ? BV : BK;
  const int capacity = val ? av.capacity : ak.capacity;
  float* const norms = val ? av.norms : ak.norms;
  const void* const xsrc = val ? av.x : ak.x;
  const int b = st / ak.n_kv_heads, kv = st - b * ak.n_kv_heads;
  const int pb = lane & 31;
  const int slot = ak.pos ? ak.pos[b] : ak.pos0;
  const int ntile = capacity / kTile;
  const int t = slot & (kTile - 1);

  // global reads first: the vector, signs, SO(4) block, and the value bytes to be merged
  float4 x;
  const size_t xi = (size_t)st * kHeadDim + 4 * pb;  // n_new == 1
  if (x_f16) {
    typedef _Float16 h4_t __attribute__((ext_vector_type(4)));
    const h4_t h = *(const h4_t*)((const _Float16*)xsrc + xi);
    x = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
  } else {
    x = *(const float4*)((const float*)xsrc + xi);
  }
  const float4 sg = *(const float4*)(ak.signs + kv * kHeadDim + 4 * pb);
  Quat ql{1.f, 0.f, 0.f, 0.f}, qr{1.f, 0.f, 0.f, 0.f};
  if (ak.so4) {
    ql = qload(ak.so4 + ((size_t)kv * 32 + pb) * 8);
    qr = qload(ak.so4 + ((size_t)kv * 32 + pb) * 8 + 4);
  }
  // value word of coordinate i = 16u + m for tile token t = 16h + 4q + r: (q*16 + m)*8 + u,
  // field 4h + r; 3-bit words are 3 bytes, 4-bit words 4 bytes
  const int q = (t >> 2) & 3, fk = 4 * (t >> 4) + (t & 3);
  uint8_t* vtile = av.codes + ((size_t)st * ntile + slot / kTile) * (kTile * 16 * BV);
  uint8_t vold[4][2];
  int vbyte[4];
  if (val) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * pb + j, u = i >> 4, m = i & 15;
      const int w = (q * 16 + m) * 8 + u;
      vbyte[j] = w * BV + (BV * fk) / 8;
      vold[j][0] = vtile[vbyte[j]];
      vold[j][1] = (BV == 3 && (BV * fk) % 8 > 5) ? vtile[vbyte[j] + 1] : 0;
    }
  }

  // norm of the group (lanes of one group: GROUP / 4 consecutive lanes of the half)
  float x0 = x.x * sg.x, x1 = x.y * sg.y, x2 = x.z * sg.z, x3 = x.w * sg.w;
  float ss = x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
#pragma unroll
  for (int m = 1; m < GROUP / 4; m <<= 1) ss += lane_xor(ss, m, lane);
  const float nrm = sqrtf(ss);
  const float inv = nrm > 0.f ? 1.0f / nrm : 0.f;
  x0 *= inv; x1 *= inv; x2 *= inv; x3 *= inv;
  // normalised Hadamard on each GROUP-block, then SO(4)
  float y0 = x0 + x1, y1 = x0 - x1, y2 = x2 + x3, y3 = x2 - x3;
  x0 = y0 + y2; x1 = y1 + y3; x2 = y0 - y2; x3 = y1 - y3;
#pragma unroll
  for (int m = 1; m < GROUP / 4; m <<= 1) {
    const bool up = (lane & m) != 0;
    const float o0 = lane_xor(x0, m, lane), o1 = lane_xor(x1, m, lane), o2 = lane_xor(x2, m, lane),
                o3 = lane_xor(x3, m, lane);
    x0 = up ? o0 - x0 : x0 + o0;
    x1 = up ? o1 - x1 : x1 + o1;
    x2 = up ? o2 - x2 : x2 + o2;
    x3 = up ? o3 - x3 : x3 + o3;
  }
  const float hsc = GROUP == 32 ? 0.17677669529663688f : 0.088388347648318440f;
  Quat v{x0 * hsc, x1 * hsc, x2 * hsc, x3 * hsc};
  if (ak.so4) v = qmul(qmul(ql, v), qconj(qr));
  const float yv[4] = {v.w, v.x, v.y, v.z};
  uint32_t code[4];
  const int nb = (1 << bits) - 1;
  constexpr int NBMAX = (1 << (BK > BV ? BK : BV)) - 1;  // constant trip count: no indexed arrays
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < NBMAX; ++k) c += k < nb && yv[j] > (val ? av.boundary[k] : ak.boundary[k]) ? 1u : 0u;
    code[j] = c;
  }

  // norms: one lane per group
  if ((pb & (GROUP / 4 - 1)) == 0) {
    const int grp = (4 * pb) / GROUP;
    norms[((size_t)st * ntile + slot / kTile) * (NG * kTile) + grp * kTile + norm_pos(t)] = nrm;
  }
  if (!val) {
    // key record: word w = coordinates 8w..8w+7 = lanes 2w (low half) and 2w + 1
    const uint32_t half = BK == 3 ? (code[0] | code[1] << 3 | code[2] << 6 | code[3] << 9)
                                  : (code[0] | code[1] << 4 | code[2] << 8 | code[3] << 12);
    const uint32_t other = __builtin_bit_cast(uint32_t, lane_xor(__builtin_bit_cast(float, half), 1, lane));
    uint8_t* rec = ak.codes + ((size_t)st * ak.capacity + slot) * (16 * BK);
    if ((pb & 1) == 0) {
      const int w = pb >> 1;
      if (BK == 3) {
        const uint32_t word = half | (other << 12);
        rec[3 * w] = (uint8_t)word;
        rec[3 * w + 1] = (uint8_t)(word >> 8);
        rec[3 * w + 2] = (uint8_t)(word >> 16);
      } else {
        *(uint32_t*)(rec + 4 * w) = half | (other << 16);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int sh = (BV * fk) % 8;
      const uint32_t fmask = ((1u << BV) - 1u) << sh, fval = code[j] << sh;
      const uint32_t cur = vold[j][0] | ((uint32_t)vold[j][1] << 8);
      const uint32_t nw = (cur & ~fmask) | fval;
      vtile[vbyte[j]] = (uint8_t)nw;
      if (BV == 3 && sh > 5) vtile[vbyte[j] + 1] = (uint8_t)(nw >> 8);
    }
  }
}

template <int BK, int BV, int GROUP, bool XF16>
__global__ __launch_bounds__(256) void append_step_kernel(const AppendArgs ak, const AppendArgs av, int batch) {
  const int st = blockIdx.x * 4 + (threadIdx.x >> 6);  // stream = b * n_kv_heads + kv
  if (st >= batch * ak.n_kv_heads) return;            // whole waves only
  append_step_wave<BK, BV, GROUP>(ak, av, st, XF16, threadIdx.x & 63);
}

// Keys and values of one step in one launch: grid z covers the keys' sequences, then the
// values' (same tiles, same rotation).
template <int BK, int BV, int GROUP, bool XF16>
__global__ __launch_bounds__(128) void append_kv_kernel(const AppendArgs ak, const AppendArgs av, int batch) {
  const int tile = ak.n_edges ? ak.edge[blockIdx.x] : blockIdx.x;
  if ((int)blockIdx.z < batch) {
    append_tile<BK, GROUP, false, XF16>(ak, blockIdx.z, blockIdx.y, tile);
  } else {
    append_tile<BV, GROUP, true, XF16>(av, blockIdx.z - batch, blockIdx.y, tile);
  }
}

// ---------------------------------------------------------------------------------------
// Shared decode pieces.

struct Unit {
  int b, kv, split, slice, h0, hs;
};

__device__ __forceinline__ Unit decode_unit(const DecodeArgs& a, bool xcd_pairs) {
  const int ns = a.n_slices;
  const int n_units = a.batch * a.n_kv_heads * a.n_splits;
  const int L = blockIdx.x;
  int unit, slice;
  if (xcd_pairs && ns > 1 && (n_units & 7) == 0) {
    // the slices of one unit get linear ids 8 apart: same XCD, dispatched together, so the
    // second one reads the shared codes from that XCD's L2
    const int g8 = L / (8 * ns), rem = L - g8 * 8 * ns;
    slice = rem >> 3;
    unit = g8 * 8 + (rem & 7);
  } else {
    unit = L / ns;
    slice = L - unit * ns;
  }
  // split-major with the last section first: the workgroups holding the newest tokens
  // (which also append them when the append is fused) are dispatched first, so they are
  // the older, first-served workgroup on their CU
  Unit u;
  const int rows = a.batch * a.n_kv_heads;
  const int rank = unit / rows, row = unit - rank * rows;
  u.split = a.n_splits - 1 - rank;
  u.kv = row % a.n_kv_heads;
  u.b = row / a.n_kv_heads;
  u.slice = slice;
  u.h0 = u.kv * a.group_size + slice * a.heads_per_slice;
  u.hs = min(a.heads_per_slice, a.group_size - slice * a.heads_per_slice);
  return u;
}

template <bool QF16>
__device__ __forceinline__ void load_queries(const DecodeArgs& a, const Unit& u, float* qbuf) {
  for (int i = threadIdx.x; i < u.hs * kHeadDim; i += blockDim.x) {
    const size_t qi = ((size_t)u.b * a.n_q_heads + u.h0 + (i >> 7)) * kHeadDim + (i & 127);
    qbuf[i] = QF16 ? (float)((const _Float16*)a.q)[qi] : ((const float*)a.q)[qi];
  }
  __syncthreads();
}

// Final per-head result o_rot[hs][128] (rotated domain, normalised) and lse in log2 units:
// either rotate back and write `out`, or write this split's partial.
__device__ __forceinline__ void write_result(const DecodeArgs& a, const Unit& u, float* obuf,
                                             const float* lse2) {
  const int tid = threadIdx.x;
  if (a.n_splits == 1) {
    if (a.lse_out && tid < u.hs) {
      a.lse_out[(size_t)u.b * a.n_q_heads + u.h0 + tid] = lse2[tid] * kLn2;
    }
    lds_rotate<false>(obuf, u.hs, a.signs + u.kv * kHeadDim, a.so4 ? a.so4 + u.kv * 256 : nullptr, a.rot_group);
    for (int i = tid; i < u.hs * kHeadDim; i += blockDim.x) {
      a.out[((size_t)u.b * a.n_q_heads + u.h0 + (i >> 7)) * kHeadDim + (i & 127)] = obuf[i];
    }
  } else {
    const size_t row0 = ((size_t)u.split * a.batch + u.b) * a.n_q_heads + u.h0;
    if (tid < u.hs) a.part_lse[row0 + tid] = lse2[tid] * kLn2;
    for (int i = tid; i < u.hs * kHeadDim; i += blockDim.x) {
      a.part_o[(row0 + (i >> 7)) * kHeadDim + (i & 127)] = obuf[i];
    }
  }
}

__device__ __forceinline__ void token_range(const DecodeArgs& a, const Unit& u, int& lo, int& hi) {
  // lengths beyond max_len (checked against the capacity on the host) are clamped, so a
  // bad device length can never move a read outside the cache
  const int T = a.seq_lens ? max(0, min(a.seq_lens[u.b] + a.len_bias, a.max_len)) : a.max_len;
  const int C = (T + a.n_splits - 1) / a.n_splits;
  lo = min(T, u.split * C);
  hi = min(T, lo + C);
}

// ---------------------------------------------------------------------------------------
// Matrix-core decode.
//
// Scores: for a 16-token tile, D[token][col] = sum_k A[token][k] B[k][col].  A holds the
// keys' codebook levels decoded through LDS tables, as fp16 numbers at the codebook's fp16
// scale s (the levels c * s are fp16 values within 3e-5 relative for 3-bit codebooks, 1e-4
// for 4-bit; the query carries 1/s).  B is the rotated query, prescaled by a power of two and
// split into fp16 high and low parts: whole-head groups put the parts in columns c and c + 8
// (one product per key operand); 32-coordinate groups use columns (group, head) and take one
// product with each part, so D holds per-group partial dots, scaled by the group norms and
// summed across the group lanes.
// Values: O[coord][col] += sum_k A[coord][k] P'[k][col] over the 32 tokens of a tile, with
// A = value codebook levels (a value word holds 8 tokens of one coordinate) and P' = p *
// value norm in fp16 (with a power-of-two range factor), taken straight from the score
// registers.  Online softmax per column.
//
// Decode tables: 3-bit codes are read through a table indexed by four codes (4096 entries
// of four fp16 levels), one for keys and values that share a codebook; 4-bit codes through
// an index of two codes (8 bits) that selects an entry of two fp16 levels, stored in 16
// copies, copy c serving lanes c, c + 16 ... with the copies of one entry side by side, so
// that the bank a lane reads is fixed by its lane number.
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c, 0,
                                                0, 0);
}


// LDS byte address of a two-code table lookup: the 2*BITS-bit field at bit `off` of d[]
// lands on bits [SH, SH + 2*BITS) of the address and the lane's copy offset fills the bits
// below (one shift or align and one bit-field insert per lookup).
template <int BITS, int SH>
__device__ __forceinline__ uint32_t pair_lds_addr(const uint32_t* d, int off, uint32_t lane_off) {
  constexpr int W = 2 * BITS;
  constexpr uint32_t mask = ((1u << W) - 1u) << SH;
  const int wi = off >> 5, sh = off & 31;
  uint32_t x;
  if (sh + W > 32) {
    x = __builtin_amdgcn_alignbit(d[wi + 1], d[wi], sh - SH);
  } else if (sh >= SH) {
    x = d[wi] >> (sh - SH);
  } else {
    x = d[wi] << (SH - sh);
  }
  return (x & mask) | lane_off;
}

__device__ __forceinline__ uint32_t quad_lds_addr(const uint32_t* d, int off) {
  const int wi = off >> 5, sh = off & 31;
  uint32_t x;
  if (sh + 12 > 32) x = __builtin_amdgcn_alignbit(d[wi + 1], d[wi], sh - 3);
  else if (sh >= 3) x = d[wi] >> (sh - 3);
  else x = d[wi] << (3 - sh);
  return x & (0xFFFu << 3);
}

template <typename T>
__device__ __forceinline__ T lds_at(const uint8_t* base, uint32_t byte_off) {
  return *(const T*)(base + byte_off);
}

template <int BK, int BV>
struct Block {
  uint32_t k0[BK], k1[BK];  // this lane's 32 key codes of tile tokens (lane&15) and 16+(lane&15)
  f32x4 kn0, kn1;           // key norms of tokens 4q'+r and 16+4q'+r (folded: kn0 only, own tile)
  uint32_t v[2 * BV];       // this lane's 8 value words
  f32x4 vn0, vn1;           // value norms, same tokens as kn
};

// Lazy softmax rescale: the running maximum is only moved when a block raises it by more
// than 2^3, so p = 2^(s - m) stays below 8.
constexpr float kRescaleLog2 = 3.0f;
// The value weight p * norm is rounded to fp16 for the matrix product.  Its range is kept by
// a power of two 2^-E folded into the softmax offset (the weights and their sum carry the
// same factor, so it cancels in the output and is added back to the lse).  E moves lazily,
// per 32-token block: when some weight of the block exceeds 2^15 or none reaches 2^-10, E is
// reset so that the block's largest weight lies in [2^3, 2^4).  Every block's largest
// weights are then normal fp16 numbers (full precision), and a weight that falls to fp16's
// subnormal range is below 2^-4 of its block's largest, with an absolute error of at most
// 2^-25.  E is clamped to [-90, 90], so that the weights and their fp32 sum stay finite at
// any cache length (value group norms up to about 2^100).
constexpr float kWeightHi = 32768.0f, kWeightLo = 0.0009765625f;  // 2^15, 2^-10
constexpr int kWeightTop = 3;                                       // largest weight to [2^3, 2^4)

// Maximum / sum over the four 16-lane rows (lanes l, l^16, l^32, l^48), with the gfx950
// row swaps: each returns the pair {x[l], x[l ^ 16]} (or ^ 32) as two values, and max and
// + do not depend on their order, so the result equals the exchange form bit for bit.
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ uint32_t rows_or(uint32_t x) {  // or over lanes l, l^16, l^32, l^48
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = a[0] | a[1];
  const auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] | b[1];
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <typename T>
__device__ __forceinline__ T load_at(const uint8_t* base, uint32_t off) {
  return *(const T*)(base + off);
}

// NW waves per workgroup: 4 with two workgroups per CU, or 8 with one (grids of at most
// one workgroup per CU, where four waves would leave one wave per SIMD).  D blocks per wave
// in the register ring: 2, or 1 where a wave holds only a few blocks (each ring slot costs
// a round of loads that the texture path processes even past the last block).
template <int BK, int BV, int NG, bool QF16, bool QUAD, int NW, int D>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void decode_mfma_kernel(const DecodeArgs a) {
  static_assert(NW == 4 || NW == 8, "four or eight waves");
  static_assert(D == 1 || D == 2, "one or two blocks in flight per wave");
  constexpr int NT = 64 * NW;
  constexpr int LDS_BUDGET = NW == 4 ? 80 * 1024 : 160 * 1024;  // per workgroup
  // whole-head groups: the query's hi and lo parts take separate columns (8 + 8), so one
  // product per key operand suffices; 32-groups: columns are (group, head), two products
  constexpr bool SPLITQ = NG == 1;
  constexpr int HPS = NG == 4 ? 4 : 8;
  // With hi/lo columns, columns c and c + 8 see the same head.  The two 16-token tiles of a
  // block are folded across that pair: after the hi + lo exchange, column c keeps tile 0's
  // scores and column c + 8 tile 1's, so the softmax runs on 4 scores per lane instead of
  // 8 duplicated ones.  Each column then carries its own running maximum and sum and its
  // own value accumulator (a partial over its tile's tokens), merged in the epilogue.
  constexpr bool FOLD = SPLITQ;
  constexpr int NPART = FOLD ? 2 * NW : NW;  // partial results per head in the epilogue
  constexpr int NP = FOLD ? 4 : 8;           // scores per lane and block
  constexpr int NEK = 256, NEV = 256;  // two-code table entries: all pairs of 4-bit codes
  constexpr int KREC = 16 * BK;
  constexpr int VTILE = kTile * 16 * BV;
  // Decode tables.  3-bit codes are read through tables indexed by four codes (12 bits, 4096
  // entries of four fp16 values, 32 KB): one read per four codes.  3-bit keys and values
  // with one codebook (QUAD) share the keys' table.  4-bit codes use two-code tables
  // [entry][copies] with 16 copies, to fit the LDS budget of two workgroups per CU at the
  // price of occasional bank conflicts.  Keys sit at 0, values at VT_AT: right after a
  // four-code value table's keys, else a power of two no smaller than either table, so that
  // a two-code value address is VT_AT | offset.
  static_assert(!QUAD || (BK == 3 && BV == 3), "the shared four-code table holds 3-bit codes");
  constexpr bool KQ = BK == 3, VQ = BV == 3 && !QUAD;  // four-code key and value tables
  constexpr int RK = 16, RV = 16;
  constexpr int SHK = 6, SHV = 6;  // log2 of a two-code entry's row bytes
  constexpr int KT_BYTES = KQ ? 32768 : NEK * RK * 4, VT_BYTES = QUAD ? 0 : VQ ? 32768 : NEV * RV * 4;
  constexpr int VT_AT = VQ ? KT_BYTES : KT_BYTES > VT_BYTES ? KT_BYTES : VT_BYTES;
  // Block ring: each wave keeps its next D blocks of 32 tokens in registers.  They
  // are read with buffer loads: the (sequence, KV head) slab in a buffer resource, the
  // block's offset in a scalar register and the lane's offset fixed, so a load costs no
  // address arithmetic, and the stream does not pass through the LDS, whose bandwidth the
  // table reads need.
  constexpr int NLD = FOLD ? 6 : 8;  // loads per block: key codes x2, value words x2, norms
  constexpr int TAB_BYTES = VT_AT + VT_BYTES;
  // the pool and the other shared arrays (query rows, staged inputs, codebook, reductions)
  // stay within the workgroup's share of the CU's 160 KB
  constexpr int STATIC_LDS = HPS * kHeadDim * 4 + (kHeadDim + 256) * 4 + 256;
  // the epilogue reuses the tables' space for the per-wave partial results
  constexpr int SCR_BYTES = NPART * HPS * (kHeadDim + 2) * 4;
  constexpr int POOL = TAB_BYTES > SCR_BYTES ? TAB_BYTES : SCR_BYTES;
  static_assert(POOL + STATIC_LDS <= LDS_BUDGET, "the workgroups of a CU share its 160 KB of LDS");
  __shared__ __attribute__((aligned(16))) uint8_t pool[POOL];
  __shared__ __attribute__((aligned(16))) float qbuf[HPS * kHeadDim];
  __shared__ __attribute__((aligned(16))) float qstage[kHeadDim + 256];  // signs, SO(4) parameters
  __shared__ float red[NW];
  __shared__ float lse2[HPS];
  const uint8_t* ktab = pool;
  float* scr = (float*)pool;

  // Every argument the prologue needs is loaded in one batch here: left to itself the
  // compiler issues the scalar argument loads one dependent round trip at a time.
  asm volatile("" ::"s"(a.kc), "s"(a.kn), "s"(a.vc), "s"(a.vn), "s"(a.q), "s"(a.seq_lens), "s"(a.signs), "s"(a.so4));
  asm volatile("" ::"s"(a.max_len), "s"(a.len_bias), "s"(a.batch), "s"(a.n_kv_heads), "s"(a.n_q_heads), "s"(a.group_size),
               "s"(a.heads_per_slice), "s"(a.n_slices), "s"(a.n_splits), "s"(a.capacity));
  asm volatile("" ::"s"(a.kscale), "s"(a.kcent[0]), "s"(a.kcent[8]), "s"(a.vcent[0]), "s"(a.vcent[8]));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const Unit u = decode_unit(a, true);
  const int col = lane & 15, qg = lane >> 4;
  const int cgrp = NG == 4 ? (col >> 2) : 0;
  const int chl = NG == 4 ? (col & 3) : (col & 7);
  const int half = FOLD ? col >> 3 : 0;  // the tile this column keeps
  const bool colok = chl < u.hs && (NG == 4 || FOLD || col < 8);
  // columns that carry no live head get p = 0: their value products multiply zeros
  const float cdead = colok ? 0.f : -INFINITY;

  // ---- token range and the first two blocks' loads, issued before the prologue
  int lo, hi;
  token_range(a, u, lo, hi);
  const int blk0 = lo / kTile, blk1 = (hi + kTile - 1) / kTile;
  const size_t sb = (size_t)u.b * a.n_kv_heads + u.kv;
  const int ntile = a.capacity / kTile;
  const uint8_t* kbase = a.kc + sb * a.capacity * KREC;
  const uint8_t* knbase = (const uint8_t*)(a.kn + sb * ntile * (NG * kTile));
  const uint8_t* vbase = a.vc + sb * ntile * VTILE;
  const uint8_t* vnbase = (const uint8_t*)(a.vn + sb * ntile * (NG * kTile));
  const uint32_t koff = (lane & 15) * KREC + qg * (4 * BK);
  // norm slots: tile token 16h + 4q + r sits at 8q + 4h + r of its group's 32
  const uint32_t noff = (cgrp * kTile + 8 * qg + 4 * half) * 4;
  const uint32_t voff = lane * (8 * BV);

  // ---- Fused append: if this workgroup's section holds the row's new position, one wave
  // quantises and writes that token first; the barrier orders its stores before every
  // read of the cache by the workgroup.  Other sections that share the token's 32-token
  // tile mask it, and the bytes it rewrites keep their other tokens' fields.
  if (a.append) {
    const int p = a.ak.pos ? a.ak.pos[u.b] : a.ak.pos0;
    if (p >= lo && p < hi) {
      if (wv == 0) append_step_wave<BK, BV, NG == 4 ? 32 : 128>(a.ak, a.av, u.b * a.n_kv_heads + u.kv, a.append_f16 != 0, lane);
      __syncthreads();
    }
  }

  // ---- The small inputs (this wave's two query rows, the signs, the SO(4) parameters) are
  // staged in LDS by direct copies issued ahead of the ring's loads, so that one counted
  // wait covers them while the ring's loads stay in flight (a register load would make the
  // compiler wait for every outstanding load).  The raw rows sit at the start of the
  // wave's own two rows of qbuf, which it later overwrites with the rotated query.
  const uint32_t qraw = lds_addr(qbuf) + wv * (2 * kHeadDim * 4);
  {
    const size_t row = (size_t)u.b * a.n_q_heads + u.h0 + 2 * wv;
    if (QF16) {
      if (lane < 32 && 2 * wv + (lane >> 4) < u.hs)
        lds_dma_addr<16, false>(qraw, (const _Float16*)a.q + row * kHeadDim + 8 * lane);
    } else {
      if (2 * wv + (lane >> 5) < u.hs) lds_dma_addr<16, false>(qraw, (const float*)a.q + row * kHeadDim + 4 * lane);
    }
    if (wv == 0 && lane < 32) lds_dma_addr<16, false>(lds_addr(qstage), a.signs + u.kv * kHeadDim + 4 * lane);
    if (wv == 1 && a.so4 != nullptr) lds_dma_addr<16, false>(lds_addr(qstage) + kHeadDim * 4, a.so4 + u.kv * 256 + 4 * lane);
  }
  // ---- then the first D blocks of this wave into its ring
  const int nblk = blk0 + wv < blk1 ? (blk1 - (blk0 + wv) + NW - 1) / NW : 0;  // this wave's blocks
  constexpr int kRsrc = 0x00020000;  // raw buffer, 32-bit data format
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, a.capacity * KREC, kRsrc);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, ntile * VTILE, kRsrc);
  const __amdgpu_buffer_rsrc_t rkn = __builtin_amdgcn_make_buffer_rsrc((void*)knbase, 0, ntile * NG * kTile * 4, kRsrc);
  const __amdgpu_buffer_rsrc_t rvn = __builtin_amdgcn_make_buffer_rsrc((void*)vnbase, 0, ntile * NG * kTile * 4, kRsrc);
  // The same slabs with no records: every access is out of range, returns zeros and moves
  // no data.  Loads past the wave's last block use them, so that every ring refill is
  // issued and the compiler's count of the loads in flight stays exact.
  const __amdgpu_buffer_rsrc_t zk = __builtin_amdgcn_make_buffer_rsrc((void*)kbase, 0, 0, kRsrc);
  const __amdgpu_buffer_rsrc_t zv = __builtin_amdgcn_make_buffer_rsrc((void*)vbase, 0, 0, kRsrc);
  const __amdgpu_buffer_rsrc_t zkn = __builtin_amdgcn_make_buffer_rsrc((void*)knbase, 0, 0, kRsrc);
  const __amdgpu_buffer_rsrc_t zvn = __builtin_amdgcn_make_buffer_rsrc((void*)vnbase, 0, 0, kRsrc);
  constexpr int kStream = 2;  // non-temporal: the cache stream is read once
  // loads block j of this wave; past the last block (clamped to it, so the offset stays
  // inside the slab) it reads nothing
  auto load_block = [&](int j) {
    const bool live = j < nblk;  // wave-uniform
    const int blk = __builtin_amdgcn_readfirstlane(blk0 + wv + NW * min(j, max(nblk - 1, 0)));
    const int ko = blk * (kTile * KREC), vo = blk * VTILE, no = blk * (NG * kTile * 4);
    const __amdgpu_buffer_rsrc_t bk = live ? rk : zk, bv = live ? rv : zv;
    const __amdgpu_buffer_rsrc_t bkn = live ? rkn : zkn, bvn = live ? rvn : zvn;
    Block<BK, BV> d;
    if (BK == 3) {
      const auto x0 = __builtin_amdgcn_raw_buffer_load_b96(bk, koff, ko, kStream);
      const auto x1 = __builtin_amdgcn_raw_buffer_load_b96(bk, koff + 16 * KREC, ko, kStream);
      d.k0[0] = x0[0]; d.k0[1] = x0[1]; d.k0[2] = x0[2];
      d.k1[0] = x1[0]; d.k1[1] = x1[1]; d.k1[2] = x1[2];
    } else {
      const auto x0 = __builtin_amdgcn_raw_buffer_load_b128(bk, koff, ko, kStream);
      const auto x1 = __builtin_amdgcn_raw_buffer_load_b128(bk, koff + 16 * KREC, ko, kStream);
      d.k0[0] = x0[0]; d.k0[1] = x0[1]; d.k0[2] = x0[2]; d.k0[BK - 1] = x0[3];
      d.k1[0] = x1[0]; d.k1[1] = x1[1]; d.k1[2] = x1[2]; d.k1[BK - 1] = x1[3];
    }
    if (BV == 3) {
      const auto y0 = __builtin_amdgcn_raw_buffer_load_b96(bv, voff, vo, kStream);
      const auto y1 = __builtin_amdgcn_raw_buffer_load_b96(bv, voff + 12, vo, kStream);
      d.v[0] = y0[0]; d.v[1] = y0[1]; d.v[2] = y0[2]; d.v[3] = y1[0]; d.v[4] = y1[1]; d.v[5] = y1[2];
    } else {
      const auto y0 = __builtin_amdgcn_raw_buffer_load_b128(bv, voff, vo, kStream);
      const auto y1 = __builtin_amdgcn_raw_buffer_load_b128(bv, voff + 16, vo, kStream);
      d.v[0] = y0[0]; d.v[1] = y0[1]; d.v[2] = y0[2]; d.v[3] = y0[3];
      d.v[4] = y1[0]; d.v[5] = y1[1]; d.v[2 * BV - 2] = y1[2]; d.v[2 * BV - 1] = y1[3];
    }
    d.kn0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(bkn, noff, no, kStream));
    d.vn0 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(bvn, noff, no, kStream));
    if (!FOLD) {
      d.kn1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(bkn, noff + 16, no, kStream));
      d.vn1 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(bvn, noff + 16, no, kStream));
    }
    return d;
  };
  Block<BK, BV> ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) ring[j] = load_block(j);

  // ---- decode tables, built while the staged inputs are in flight.  The codebook's fp16
  // values (kernel arguments at constant offsets: scalar loads) go to lanes 0-15 of one
  // register (lane c selects value c), and each thread takes its entries' values by lane
  // exchange.
  int kcb = 0, vcb = 0;
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    if (lane == c) {
      kcb = (int)f16_bits((_Float16)(a.kcent[c] * a.kscale));
      vcb = (int)f16_bits((_Float16)(QUAD ? a.vcent[c] * a.kscale : a.vcent[c]));
    }
  }
  // A four-code table: thread tid owns the entries whose two low codes are (tid >> 3) & 7,
  // tid & 7; wave wv takes 64 / NW of the 64 pairs of high codes.  The low half of a
  // thread's entries is fixed, and each step writes 64 consecutive entries.
  auto quad_table = [&](uint8_t* base, int cb) {
    const uint32_t lo = (uint32_t)__shfl(cb, tid & 7) | ((uint32_t)__shfl(cb, (tid >> 3) & 7) << 16);
#pragma unroll
    for (int j = 0; j < 64 / NW; ++j) {
      const int hc = wv * (64 / NW) + j, c2 = hc & 7, c3 = hc >> 3;
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane(cb, c2) | ((uint32_t)__builtin_amdgcn_readlane(cb, c3) << 16);
      ((uint2*)base)[(tid & 63) | (c2 << 6) | (c3 << 9)] = make_uint2(lo, hi);
    }
  };
  if (KQ) {
    quad_table(pool, kcb);
  } else {
    for (int i = tid; i < NEK * RK; i += NT) {
      const int e = i / RK;
      ((uint32_t*)pool)[i] = (uint32_t)__shfl(kcb, e & ((1 << BK) - 1)) | ((uint32_t)__shfl(kcb, e >> BK) << 16);
    }
  }
  if (VQ) quad_table(pool + VT_AT, vcb);
  for (int i = tid; i < (BV == 3 ? 0 : NEV * RV); i += NT) {
    const int e = i / RV;
    ((uint32_t*)(pool + VT_AT))[i] = (uint32_t)__shfl(vcb, e & ((1 << BV) - 1)) | ((uint32_t)__shfl(vcb, e >> BV) << 16);
  }
  // the staged inputs (copied before the ring's D blocks) have landed
  vm_wait<D * NLD>();
  __syncthreads();

  // ---- rotated, scaled query (log2 units) with a power-of-two prescale into fp16 range
  float mx = 0.f;
  {
    const QueryLane qlane = query_staged<QF16>((const uint8_t*)qbuf + wv * (2 * kHeadDim * 4), qstage, a.so4 != nullptr,
                                               u.hs, wv, lane);
    float4 r = query_rotate<NG == 4 ? 32 : 128>(qlane, a.so4 != nullptr, lane);
    const float qsc = a.scale_log2 / a.kscale;
    r.x *= qsc; r.y *= qsc; r.z *= qsc; r.w *= qsc;
    if (qlane.live) {
      *(float4*)(qbuf + (2 * wv + (lane >> 5)) * kHeadDim + 4 * (lane & 31)) = r;
      mx = fmaxf(fmaxf(fabsf(r.x), fabsf(r.y)), fmaxf(fabsf(r.z), fabsf(r.w)));
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, lane_xor(mx, o, lane));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red[w]);
  int ex = 0;
  if (mx > 0.f && mx < INFINITY) (void)frexpf(mx, &ex);
  const float qs = ldexpf(1.f, 14 - ex), qinv = ldexpf(1.f, ex - 14);

  // B operands.  Key operand f of lane group q holds codes of coordinates 32q + 8f + j
  // (j = 0..7); "hi" columns see q_hi, "lo" columns q_lo (whole-head groups), or every
  // column sees q_hi in one product and q_lo in a second (32-groups).
  u32x4 B1[4], B2[4];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    u32x4 bh, bl;
    const int head = NG == 4 ? chl : (col & 7);
    const bool live = head < u.hs && (NG == 1 || cgrp == qg);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      float x0 = 0.f, x1 = 0.f;
      if (live) {
        const float* src = qbuf + head * kHeadDim + 32 * qg + 8 * f + 2 * p;
        x0 = src[0] * qs;
        x1 = src[1] * qs;
      }
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      bh[p] = f16_bits(h0) | (f16_bits(h1) << 16);
      bl[p] = f16_bits((_Float16)(x0 - (float)h0)) | (f16_bits((_Float16)(x1 - (float)h1)) << 16);
    }
    if (SPLITQ) {
      B1[f] = col < 8 ? bh : bl;
    } else {
      B1[f] = bh;
      B2[f] = bl;
    }
  }

  const uint32_t klane = (lane & (RK - 1)) << 2, vlane = VT_AT | ((lane & (RV - 1)) << 2);
  auto key_operand = [&](const uint32_t* kk, int f) {
    u32x4 r;
    if (KQ) {
      const uint2 x0 = lds_at<uint2>(pool, quad_lds_addr(kk, 24 * f)), x1 = lds_at<uint2>(pool, quad_lds_addr(kk, 24 * f + 12));
      return u32x4{x0.x, x0.y, x1.x, x1.y};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = lds_at<uint32_t>(ktab, pair_lds_addr<BK, SHK>(kk, 8 * BK * f + 2 * BK * i, klane));
    return r;
  };

  // running maximum (prescaled units), sum, the rescale bound m_run + 2^3 (prescaled) and
  // the exponent offset -m_run - ve (log2 units) plus the dead-column mask; ve is the
  // wave-uniform exponent E of the value weights' scale 2^-E
  float m_run = -INFINITY, l_run = 0.f, thr = -INFINITY, nmq = cdead;
  float ve = 0.f;
  f32x4 O[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) O[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto process = [&](const Block<BK, BV>& cb, int blk) {
    // Table reads are issued in batches ahead of their consumers so that LDS latency
    // overlaps matrix-core and vector work: all key operands of tile 0, then tile 1's
    // while tile 0 multiplies, then every value operand before the softmax arithmetic.
    u32x4 ka[4], kb[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) ka[f] = key_operand(cb.k0, f);
    f32x4 D0 = {0.f, 0.f, 0.f, 0.f}, D1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      kb[f] = key_operand(cb.k1, f);
      D0 = mfma16(ka[f], B1[f], D0);
      if (!SPLITQ) D0 = mfma16(ka[f], B2[f], D0);
    }
    u32x4 va[8];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      D1 = mfma16(kb[f], B1[f], D1);
      if (!SPLITQ) D1 = mfma16(kb[f], B2[f], D1);
    }
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (BV == 3) {
        const uint8_t* vt = pool + (QUAD ? 0 : VT_AT);
        const uint2 x0 = lds_at<uint2>(vt, quad_lds_addr(cb.v, 24 * f)), x1 = lds_at<uint2>(vt, quad_lds_addr(cb.v, 24 * f + 12));
        va[f] = u32x4{x0.x, x0.y, x1.x, x1.y};
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) va[f][j] = lds_at<uint32_t>(pool, pair_lds_addr<BV, SHV>(cb.v, 8 * BV * f + 2 * BV * j, vlane));
      }
    }
    // raw scores (units of the prescaled query).  Unfolded: tokens 16h + 4q' + r in slot
    // k = 4h + r.  Folded: tokens 16*half + 4q' + r in slot r.
    float x[NP];
    if (FOLD) {
      // column c < 8 holds tile 0's hi part and needs its lo part from column c + 8;
      // column c + 8 holds tile 1's lo part and needs its hi part from column c
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float own = half ? D1[r] : D0[r], send = half ? D0[r] : D1[r];
        x[r] = (own + dpp<0x128>(send)) * cb.kn0[r];  // row_ror:8
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        float d = k < 4 ? D0[k] : D1[k - 4];
        const float n = k < 4 ? cb.kn0[k] : cb.kn1[k - 4];
        if (NG == 4) {
          d *= n;
          d += dpp<0x124>(d);  // row_ror:4
          d += dpp<0x128>(d);  // row_ror:8
        } else {
          d = (d + dpp<0x128>(d)) * n;  // hi + lo columns
        }
        x[k] = d;
      }
    }
    const int t0 = blk * kTile;
    const bool edge = t0 < lo || t0 + kTile > hi;  // wave-uniform
    // the value group norms of this lane's scores (a token's norm of its coordinate group)
    float vn[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) vn[k] = FOLD || k < 4 ? cb.vn0[k & 3] : cb.vn1[k - 4];
    if (edge) {
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        const int t = FOLD ? t0 + 16 * half + 4 * qg + k : t0 + 16 * (k >> 2) + 4 * qg + (k & 3);
        if (t < lo || t >= hi) {
          x[k] = -INFINITY;
          vn[k] = 0.f;  // masked slots may hold undefined norms
        }
      }
    }
    // Lazy maximum: while no score of the block exceeds the column's running maximum by
    // more than 2^kRescaleLog2 (thr is that bound in prescaled units), p stays below it and
    // nothing needs to be reduced across the lanes; only when some lane sees a larger
    // score is the block maximum formed and the column rescaled.
    float lm = x[0];
#pragma unroll
    for (int k = 1; k < NP; ++k) lm = fmaxf(lm, x[k]);
    if (__builtin_amdgcn_ballot_w64(lm > thr) != 0) {
      const float bm = rows_max(lm);
      const float mnew = bm > thr ? bm : m_run;
      const float al = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - mnew) * qinv);
#pragma unroll
      for (int i = 0; i < 8; ++i) O[i] *= al;
      l_run *= al;
      m_run = mnew;
      thr = m_run + kRescaleLog2 * qs;
      nmq = (m_run == -INFINITY ? 0.f : -m_run * qinv) - ve + cdead;
    }
    float p[NP], lp[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      lp[k] = fmaf(x[k], qinv, nmq);  // log2 of the weight, 2^-E included
      p[k] = __builtin_amdgcn_exp2f(lp[k]);
      l_run += p[k];
    }
    float pv[NP];
    float pm = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      pv[k] = p[k] * vn[k];
      pm = fmaxf(pm, pv[k]);
    }
    // The value weights' scale: rescaled only when a weight of the block would leave fp16's
    // range (above 2^15) or when every weight of the block is below 2^-10.  The block's
    // largest weight is found from log2 p + log2 norm, which cannot overflow.
    if (__builtin_amdgcn_ballot_w64(pm > kWeightHi) != 0 || __builtin_amdgcn_ballot_w64(pm >= kWeightLo) == 0) {
      float wl = -INFINITY;
#pragma unroll
      for (int k = 0; k < NP; ++k) wl = fmaxf(wl, vn[k] > 0.f ? lp[k] + __log2f(vn[k]) : -INFINITY);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) wl = fmaxf(wl, lane_xor(wl, o, lane));
      wl = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wl)));
      if (wl > -INFINITY) {  // some weight is nonzero
        const int en = min(max((int)ve + (int)floorf(wl) - kWeightTop, -90), 90);
        const float al = ldexpf(1.f, (int)ve - en);
#pragma unroll
        for (int i = 0; i < 8; ++i) O[i] *= al;
        l_run *= al;  // this block's weights included
#pragma unroll
        for (int k = 0; k < NP; ++k) pv[k] *= al;
        nmq += ve - (float)en;
        ve = (float)en;
      }
    }
    typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
    u32x4 bp;
    if (FOLD) {
      // this column's tile takes K slots 4*half .. 4*half + 3; the other tile's are zero
      const uint32_t c01 = __builtin_bit_cast(uint32_t, h2_t{(_Float16)pv[0], (_Float16)pv[1]});
      const uint32_t c23 = __builtin_bit_cast(uint32_t, h2_t{(_Float16)pv[2], (_Float16)pv[3]});
      bp[0] = half ? 0u : c01;
      bp[1] = half ? 0u : c23;
      bp[2] = half ? c01 : 0u;
      bp[3] = half ? c23 : 0u;
    } else {
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const h2_t hv = {(_Float16)pv[2 * pr], (_Float16)pv[2 * pr + 1]};
        bp[pr] = __builtin_bit_cast(uint32_t, hv);
      }
    }
#pragma unroll
    for (int w = 0; w < 8; ++w) O[w] = mfma16(va[w], bp, O[w]);
  };

  // Block j is processed from ring slot j % D, which then takes block j + D: with D = 2 the
  // next block loads during the arithmetic.
  for (int j0 = 0; j0 < nblk; j0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int j = j0 + s;
      if (j < nblk) process(ring[s], blk0 + wv + NW * j);
      ring[s] = load_block(j + D);
    }
  }

  // ---- combine the partials of the workgroup: one per wave, or per wave and tile when
  // folded (scores in prescaled units -> log2 units)
  const float lt = rows_sum(l_run);
  // the weights and their sum carry 2^-E: the partial's log2 maximum takes E back
  const float m2 = m_run == -INFINITY ? -INFINITY : m_run * qinv + ve;
  __syncthreads();                          // every wave is done with the tables
  const int part = FOLD ? 2 * wv + half : wv;
  float* so = scr;                          // [NPART][HPS][128]
  float* sm = so + NPART * HPS * kHeadDim;  // [NPART][HPS]
  float* sl = sm + NPART * HPS;
  if (colok) {
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      if (NG == 1 || (w >> 1) == cgrp) {
#pragma unroll
        for (int r = 0; r < 4; ++r) so[(part * HPS + chl) * kHeadDim + 16 * w + 4 * qg + r] = O[w][r];
      }
    }
    if (qg == 0 && cgrp == 0) {
      sm[part * HPS + chl] = m2;
      sl[part * HPS + chl] = lt;
    }
  }
  __syncthreads();
  for (int i = tid; i < u.hs * kHeadDim; i += NT) {
    const int hl = i >> 7, c = i & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NPART; ++w) M = fmaxf(M, sm[w * HPS + hl]);
    const float mu = M == -INFINITY ? 0.f : M;
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NPART; ++w) {
      const float f = __builtin_amdgcn_exp2f(sm[w * HPS + hl] - mu);
      L += sl[w * HPS + hl] * f;
      acc += so[(w * HPS + hl) * kHeadDim + c] * f;
    }
    const float o = L > 0.f ? (QUAD ? acc / (L * a.kscale) : acc / L) : 0.f;
    const float lse = L > 0.f ? M + __log2f(L) : -INFINITY;
    if (a.n_splits > 1) {
      // a section's partial stays in the rotated domain: written straight from here
      const size_t row = ((size_t)u.split * a.batch + u.b) * a.n_q_heads + u.h0 + hl;
      a.part_o[row * kHeadDim + c] = o;
      if (c == 0) a.part_lse[row] = lse * kLn2;
    } else {
      qbuf[i] = o;
      if (c == 0) lse2[hl] = lse;
    }
  }
  if (a.n_splits == 1) {
    __syncthreads();
    write_result(a, u, qbuf, lse2);
  }
}


// ---------------------------------------------------------------------------------------
// Append of whole tiles by matrix cores (fp16 vectors, one start position for all rows).
//
// The rotation of one KV head is a fixed 128 x 128 matrix R applied to the raw vector (the
// norm divides afterwards): R[o][k] = s[k] / sqrt(g) * sum_j M[o][j] H[j][k], with s the
// sign flips, H the Sylvester Hadamard on each g-block and M the SO(4) block matrix
// (identity without SO(4)).  A tile of 32 tokens is one product of R with the tile's
// vectors.  The fp16 vectors are exact operands; R is split into fp16 high and low parts,
// so two products give the rotated values to about fp32 accuracy (without SO(4) blocks R's
// entries are +-1/sqrt(g): stored as +-1 they are exact and one product suffices).  The
// workgroup builds R
// once, in LDS, already in matrix-core operand order (16 x 32 blocks of 64 lanes x 16
// bytes: conflict-free reads; 32-groups keep only the diagonal blocks).  Each wave then
// takes whole tiles on its own, loading the next tile's vectors during this one's
// arithmetic.  A token's norm comes from the same operands (fp16 pair dot products, fp32
// sums).  Codes are counted against the boundaries with the quantiser's odd symmetry (the
// boundaries are exactly symmetric, the middle one exactly zero): the sign, then a binary
// search of the upper half's boundaries on |y|.  Keys take the products as (output, token), so a lane holds four
// consecutive coordinates of one token and the four lane rows together a 96-bit chunk of
// its record; values take them as (token, output), so a lane holds, across both token
// blocks, the eight tokens of one stored value word.
// Number of the quantiser's upper-half boundaries (sorted, NU = 3 or 7) strictly below
// a >= 0, by binary search: two or three comparisons.
template <int NU>
__device__ __forceinline__ uint32_t upper_count(float a, const float* ub) {
  if (NU == 3) {
    const bool c1 = a > ub[1];
    const bool c2 = a > (c1 ? ub[2] : ub[0]);
    return (c1 ? 2u : 0u) + (c2 ? 1u : 0u);
  } else {
    const bool c1 = a > ub[3];
    const bool c2 = a > (c1 ? ub[5] : ub[1]);
    const bool c3 = a > (c1 ? (c2 ? ub[6] : ub[4]) : (c2 ? ub[2] : ub[0]));
    return (c1 ? 4u : 0u) + (c2 ? 2u : 0u) + (c3 ? 1u : 0u);
  }
}

template <int BITS, int GROUP, bool VALUES, int NWV, bool EXACT>
__device__ __forceinline__ void append_mfma_tiles(const AppendArgs& a, int b, int h, int j_begin, int j_end,
                                                  uint8_t* rlds) {
  constexpr int NG = kHeadDim / GROUP;
  constexpr int NKS = GROUP == 128 ? 4 : 1;  // K steps of 32 per output block
  constexpr int HALF = 1 << (BITS - 1);     // codes of the quantiser's upper half
  constexpr int NU = HALF - 1;               // boundaries above zero
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, qg = lane >> 4;
  const size_t stream = (size_t)b * a.n_kv_heads + h;
  const int ntile = a.capacity / kTile;
  const float gscale = GROUP == 32 ? 0.17677669529663688f : 0.088388347648318440f;
  // EXACT (no SO(4) blocks): the rotation's entries are +-1/sqrt(g); stored as +-1 they are
  // exact fp16 operands (the low parts vanish and their products are skipped), and 1/sqrt(g)
  // joins the 1/norm scale of the results.
  const float rscale = EXACT ? 1.f : gscale, yscale = EXACT ? gscale : 1.f;
  float ub[NU];
#pragma unroll
  for (int k = 0; k < NU; ++k) ub[k] = a.boundary[HALF + k];

  // ---- R in LDS: operand (part, ob, s) at ((part * 8 + ob) * NKS + s) * 1 KB, lane l's 16 bytes
  // holding R[16 ob + (l & 15)][32 ks + 8 (l >> 4) + 0..7] (ks = s, or ob >> 1 for 32-groups)
  for (int op = wv; op < 8 * NKS; op += NWV) {
    const int ob = op / NKS, ks = GROUP == 128 ? op % NKS : ob >> 1;
    const int o = 16 * ob + col;
    float mrow[4];  // row o & 3 of the SO(4) matrix of o's 4-block
    if (a.so4 != nullptr) {
      const float* qp = a.so4 + ((size_t)h * 32 + (o >> 2)) * 8;
      const Quat ql = qload(qp), qrc = qconj(qload(qp + 4));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const Quat e{c == 0 ? 1.f : 0.f, c == 1 ? 1.f : 0.f, c == 2 ? 1.f : 0.f, c == 3 ? 1.f : 0.f};
        const Quat r = qmul(qmul(ql, e), qrc);
        const int i = o & 3;
        mrow[c] = i == 0 ? r.w : i == 1 ? r.x : i == 2 ? r.y : r.z;
      }
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) mrow[c] = c == (o & 3) ? 1.f : 0.f;
    }
    u32x4 hi, lo;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint32_t hw = 0, lw = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int k = 32 * ks + 8 * qg + 2 * p + e;
        float r = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int jj = (o & ~3) + c;
          r += (__builtin_popcount(jj & k & (GROUP - 1)) & 1) ? -mrow[c] : mrow[c];
        }
        r *= a.signs[h * kHeadDim + k] * rscale;
        const _Float16 rh = (_Float16)r;
        hw |= f16_bits(rh) << (16 * e);
        lw |= f16_bits((_Float16)(r - (float)rh)) << (16 * e);
      }
      hi[p] = hw;
      lo[p] = lw;
    }
    *(u32x4*)(rlds + (0 * 8 * NKS + op) * 1024 + 16 * lane) = hi;
    *(u32x4*)(rlds + (1 * 8 * NKS + op) * 1024 + 16 * lane) = lo;
  }
  __syncthreads();
  auto r_op = [&](int part, int ob, int s) {
    return *(const u32x4*)(rlds + ((part * 8 + ob) * NKS + s) * 1024 + 16 * lane);
  };

  // ---- this stream's vectors: fp16 rows of 256 bytes; lane (col, qg) reads token
  // 16 tb + col, bytes 64 ks + 16 qg .. + 15 of its row
  constexpr int kRsrc = 0x00020000;
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc((void*)((const uint8_t*)a.x + stream * a.n_new * 256), 0, a.n_new * 256, kRsrc);
  const uint32_t xoff = col * 256 + 16 * qg;
  auto load_tile = [&](int j, u32x4 (&B)[2][4]) {
    const int so = __builtin_amdgcn_readfirstlane((min(j, j_end - 1) * kTile - a.pos0) * 256);
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        B[tb][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, xoff + 4096 * tb + 64 * ks, so, 2));
  };

  auto tile_step = [&](int j, const u32x4 (&B)[2][4]) {
    // norms of tokens 16 tb + col (one per 32-group)
    float inv[2][NG];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (GROUP == 128 || ks == g) {
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const uint32_t w = B[tb][ks][p];  // (a bit cast of the vector element itself reads element 0)
              const h2_t v = __builtin_bit_cast(h2_t, w);
              if (p & 1) s1 = __builtin_amdgcn_fdot2(v, v, s1, false);
              else s0 = __builtin_amdgcn_fdot2(v, v, s0, false);
            }
          }
        }
        const float nrm = sqrtf(rows_sum(s0 + s1));
        inv[tb][g] = nrm > 0.f ? yscale / nrm : 0.f;
        if (qg == g % 4)  // one row of lanes per group writes
          a.norms[(stream * ntile + j) * (NG * kTile) + g * kTile + norm_pos(16 * tb + col)] = nrm;
      }
    }
    // values: the norm of token 16 tb + 4 qg + i lives in lane 4 qg + i
    float vinv[2][NG][4];
    if (VALUES) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
          for (int i = 0; i < 4; ++i) vinv[tb][g][i] = __shfl(inv[tb][g], 4 * qg + i);
    }
    const int t0 = j * kTile;
    uint32_t vword[8];
    uint32_t kf[2][2];  // keys: fields of output blocks 2c, 2c + 1 for both token blocks
#pragma unroll
    for (int ob = 0; ob < 8; ++ob) {
      const int g = GROUP == 32 ? ob >> 1 : 0;
      // R's operands are read per output block: hoisted out of the loops they would hold
      // every block's operands in registers at once
      asm volatile("" ::: "memory");
      u32x4 ahi[NKS], alo[NKS];
#pragma unroll
      for (int s2 = 0; s2 < NKS; ++s2) {
        ahi[s2] = r_op(0, ob, s2);
        if (!EXACT) alo[s2] = r_op(1, ob, s2);
      }
      vword[ob] = 0u;
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s2 = 0; s2 < NKS; ++s2) {
          const int ks = GROUP == 128 ? s2 : ob >> 1;
          if (VALUES) {
            acc = mfma16(B[tb][ks], ahi[s2], acc);
            if (!EXACT) acc = mfma16(B[tb][ks], alo[s2], acc);
          } else {
            acc = mfma16(ahi[s2], B[tb][ks], acc);
            if (!EXACT) acc = mfma16(alo[s2], B[tb][ks], acc);
          }
        }
        uint32_t f = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float y = acc[i] * (VALUES ? vinv[tb][g][i] : inv[tb][g]);
          // The sign, then the count of upper-half boundaries strictly below |y|.  A negative
          // value exactly on a boundary thus takes the code above it, where the compare-count
          // rule gives the one below; making that count strict too (|y| one ulp up when
          // y <= 0) cost 13% of the kernel's time, for a tie that real-valued inputs reach
          // with probability zero (zero vectors, y = 0, keep the rule's code).
          uint32_t m;
          if (VALUES && NU == 7) {  // (the search's selects cost 4-bit value words too many registers)
            m = 0;
#pragma unroll
            for (int k = 0; k < NU; ++k) m += fabsf(y) > ub[k] ? 1u : 0u;
          } else {
            m = upper_count<NU>(fabsf(y), ub);
          }
          const uint32_t code = (y > 0.f ? (uint32_t)HALF : (uint32_t)(HALF - 1)) ^ m;
          f |= code << (BITS * i);
        }
        if (VALUES) vword[ob] |= f << (4 * BITS * tb);
        else kf[ob & 1][tb] = f;
      }
      if (!VALUES && (ob & 1)) {
        // chunk c = ob / 2 (coordinates 32 c .. + 31) of token 16 tb + col: lane row qg holds
        // coordinates 4 qg .. + 3 of both output blocks; place them and merge the four rows
        const int c = ob >> 1;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          // chunk bit of coordinate 32 c + m: BITS * m.  3-bit: the second block starts at bit
          // 48, taken relative to bit 32; 4-bit: at bit 64, relative to bit 64
          const uint64_t p0 = (uint64_t)kf[0][tb] << (BITS * 4 * qg);
          const uint64_t p1 = (uint64_t)kf[1][tb] << (BITS == 3 ? 12 * qg + 16 : 16 * qg);
          uint32_t w0 = (uint32_t)p0, w1, w2, w3 = 0u;
          if (BITS == 3) {
            w1 = (uint32_t)(p0 >> 32) | (uint32_t)p1;
            w2 = (uint32_t)(p1 >> 32);
          } else {
            w1 = (uint32_t)(p0 >> 32);
            w2 = (uint32_t)p1;
            w3 = (uint32_t)(p1 >> 32);
          }
          w0 = rows_or(w0); w1 = rows_or(w1); w2 = rows_or(w2);
          if (BITS == 4) w3 = rows_or(w3);
          if (qg == 0) {
            uint32_t* o = (uint32_t*)(a.codes + (stream * a.capacity + t0 + 16 * tb + col) * (16 * BITS) + c * (4 * BITS));
            if (BITS == 3) {
              o[0] = w0; o[1] = w1; o[2] = w2;
            } else {
              *(uint4*)o = make_uint4(w0, w1, w2, w3);
            }
          }
        }
      }
    }
    if (VALUES) {  // words u = 0..7 of (q, m) = (qg, col): consecutive in the tile
      uint32_t* vt = (uint32_t*)(a.codes + (stream * ntile + j) * (kTile * 16 * BITS) + (qg * 16 + col) * 8 * BITS);
      if (BITS == 3) {
#pragma unroll
        for (int e = 0; e < 6; ++e) {  // dword e = bits 32 e .. + 31 of the 8 x 24-bit words
          const int bit = 32 * e, wi = bit / 24, sh = bit % 24;  // sh in {0, 8, 16}
          vt[e] = (vword[wi] >> sh) | (vword[wi + 1] << (24 - sh));
        }
      } else {
        *(uint4*)vt = make_uint4(vword[0], vword[1], vword[2], vword[3]);
        *(uint4*)(vt + 4) = make_uint4(vword[4], vword[5], vword[6], vword[7]);
      }
    }
  };

  // this wave's tiles j_begin + wv, + NWV, ...: two in registers, the next one loading
  // during the arithmetic (past the last the load repeats it: every load is issued, so the
  // compiler's count of loads in flight stays exact)
  u32x4 B0[2][4], B1[2][4];
  const int jw = j_begin + wv;
  load_tile(jw, B0);
  for (int j = jw; j < j_end; j += 2 * NWV) {
    load_tile(j + NWV, B1);
    tile_step(j, B0);
    load_tile(j + 2 * NWV, B0);
    if (j + NWV < j_end) tile_step(j + NWV, B1);
  }
}

// Waves per workgroup and workgroups per CU: whole-head groups keep 64 KB of R in LDS (two
// workgroups of six waves), 32-groups 16 KB (three of four); three waves per SIMD either way.
template <int GROUP>
struct MfmaAppendShape {
  static constexpr int kWaves = GROUP == 128 ? 6 : 4;
  static constexpr int kPerCu = GROUP == 128 ? 2 : 3;
  static constexpr int kLds = 2 * 8 * (GROUP == 128 ? 4 : 1) * 1024;
};

// Whole tiles [j0, j0 + n_full) of every (sequence, KV head), per_wg tiles per workgroup.
template <int BITS, int GROUP, bool VALUES, bool EXACT>
__global__ __launch_bounds__(64 * MfmaAppendShape<GROUP>::kWaves, MfmaAppendShape<GROUP>::kPerCu) void append_mfma_kernel(
    const AppendArgs a, int j0, int n_full, int per_wg) {
  using S = MfmaAppendShape<GROUP>;
  __shared__ __attribute__((aligned(16))) uint8_t rlds[S::kLds];
  const int jb = j0 + blockIdx.x * per_wg;
  append_mfma_tiles<BITS, GROUP, VALUES, S::kWaves, EXACT>(a, blockIdx.z, blockIdx.y, jb, min(jb + per_wg, j0 + n_full),
                                                           rlds);
}
// Keys (grid z < batch) and values in one launch.
template <int BK, int BV, int GROUP, bool EXACT>
__global__ __launch_bounds__(64 * MfmaAppendShape<GROUP>::kWaves, MfmaAppendShape<GROUP>::kPerCu) void append_mfma_kv_kernel(
    const AppendArgs ak, const AppendArgs av, int batch, int j0, int n_full, int per_wg) {
  using S = MfmaAppendShape<GROUP>;
  __shared__ __attribute__((aligned(16))) uint8_t rlds[S::kLds];
  const int jb = j0 + blockIdx.x * per_wg, je = min(jb + per_wg, j0 + n_full);
  if ((int)blockIdx.z < batch) append_mfma_tiles<BK, GROUP, false, S::kWaves, EXACT>(ak, blockIdx.z, blockIdx.y, jb, je, rlds);
  else append_mfma_tiles<BV, GROUP, true, S::kWaves, EXACT>(av, blockIdx.z - batch, blockIdx.y, jb, je, rlds);
}

// ---------------------------------------------------------------------------------------
// Vector (fp32) decode: token-parallel scores, dimension-parallel value sum, 64-token
// steps.  Plain arithmetic; the cross-check for the matrix-core schedule and the fallback
// for shapes it does not take.
template <int BK, int BV, int NG, bool QF16>
__global__ __launch_bounds__(256) void decode_vec_kernel(const DecodeArgs a) {
  constexpr int MAXH = 16;
  constexpr int KREC = 16 * BK;
  __shared__ float qbuf[MAXH * kHeadDim];
  __shared__ float cbk[16], cbv[16];
  __shared__ float ps[MAXH][4][64];
  __shared__ float pw[MAXH][64];
  __shared__ float hm[MAXH], hsum[MAXH], halpha[MAXH];
  __shared__ float oacc[2][MAXH][kHeadDim];
  __shared__ float lse2[MAXH];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const Unit u = decode_unit(a, false);
  if (tid < 16) {
    cbk[tid] = a.kcent[tid];
    cbv[tid] = a.vcent[tid];
  }
  if (tid < MAXH) {
    hm[tid] = -INFINITY;
    hsum[tid] = 0.f;
  }
  load_queries<QF16>(a, u, qbuf);
  lds_rotate<true>(qbuf, u.hs, a.signs + u.kv * kHeadDim, a.so4 ? a.so4 + u.kv * 256 : nullptr, a.rot_group);
  for (int i = tid; i < u.hs * kHeadDim; i += 256) qbuf[i] *= a.scale_log2;
  __syncthreads();

  int lo, hi;
  token_range(a, u, lo, hi);
  const size_t sb = (size_t)u.b * a.n_kv_heads + u.kv;
  const int ntile = a.capacity / kTile;
  const int i_coord = tid & 127, half = tid >> 7;
  float acc[MAXH];
#pragma unroll
  for (int h = 0; h < MAXH; ++h) acc[h] = 0.f;

  for (int c0 = (lo / kTile) * kTile; c0 < hi; c0 += 64) {
    // phase 1: partial scores, thread (token, quarter of the coordinates)
    {
      const int t = lane, part = wv, tok = c0 + t;
      float pp[MAXH];
#pragma unroll
      for (int h = 0; h < MAXH; ++h) pp[h] = 0.f;
      if (tok >= lo && tok < hi) {
        uint32_t d[BK];
        const uint32_t* kp = (const uint32_t*)(a.kc + (sb * a.capacity + tok) * KREC + part * 4 * BK);
#pragma unroll
        for (int j = 0; j < BK; ++j) d[j] = kp[j];
        float cv[32];
#pragma unroll
        for (int e = 0; e < 32; ++e) cv[e] = cbk[field<BK>(d, BK * e)];
        const float nk = a.kn[(sb * ntile + tok / kTile) * (NG * kTile) + (NG == 4 ? part : 0) * kTile +
                              norm_pos(tok & (kTile - 1))];
#pragma unroll
        for (int h = 0; h < MAXH; ++h) {
          if (h < u.hs) {
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 32; ++e) s = fmaf(qbuf[h * kHeadDim + 32 * part + e], cv[e], s);
            pp[h] = s * nk;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < MAXH; ++h)
        if (h < u.hs) ps[h][part][t] = pp[h];
    }
    __syncthreads();
    // phase 2: per-head online softmax over the 64 tokens
    for (int h = wv; h < u.hs; h += 4) {
      const int tok = c0 + lane;
      float s = ps[h][0][lane] + ps[h][1][lane] + ps[h][2][lane] + ps[h][3][lane];
      s = (tok >= lo && tok < hi) ? s : -INFINITY;
      float bm = s;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o));
      const float mold = hm[h];
      const float mnew = fmaxf(mold, bm);
      const float al = mnew > mold ? __builtin_amdgcn_exp2f(mold - mnew) : 1.f;
      const float mu = mnew == -INFINITY ? 0.f : mnew;
      const float p = __builtin_amdgcn_exp2f(s - mu);
      float psum = p;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) psum += __shfl_xor(psum, o);
      pw[h][lane] = p;
      if (lane == 0) {
        hm[h] = mnew;
        hsum[h] = hsum[h] * al + psum;
        halpha[h] = al;
      }
    }
    __syncthreads();
    // phase 3: thread (coordinate, tile half) accumulates its coordinate over 32 tokens
    {
#pragma unroll
      for (int h = 0; h < MAXH; ++h)
        if (h < u.hs) acc[h] *= halpha[h];
      const int tile = c0 / kTile + half;
      const int m = i_coord & 15, mu = i_coord >> 4;
      const uint8_t* tbase = a.vc + (sb * ntile + tile) * (kTile * 16 * BV);
      const float* nbase = a.vn + (sb * ntile + tile) * (NG * kTile) + (NG == 4 ? (i_coord >> 5) : 0) * kTile;
      for (int t32 = 0; t32 < kTile; ++t32) {
        const int tok = tile * kTile + t32;
        if (tok < lo || tok >= hi) continue;
        const int q = (t32 >> 2) & 3, kap = 4 * (t32 >> 4) + (t32 & 3);
        const int bit = ((q * 16 + m) * 8 + mu) * (8 * BV) + BV * kap;
        // a 3-bit field may straddle two bytes of its word; read the second only then, so
        // the read never leaves the word
        uint32_t two = tbase[bit >> 3];
        if ((bit & 7) + BV > 8) two |= (uint32_t)tbase[(bit >> 3) + 1] << 8;
        const uint32_t code = (two >> (bit & 7)) & ((1u << BV) - 1u);
        const float f = cbv[code] * nbase[norm_pos(t32)];
        const int pt = half * kTile + t32;
#pragma unroll
        for (int h = 0; h < MAXH; ++h)
          if (h < u.hs) acc[h] = fmaf(pw[h][pt], f, acc[h]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int h = 0; h < MAXH; ++h)
    if (h < u.hs) oacc[half][h][i_coord] = acc[h];
  __syncthreads();
  for (int i = tid; i < u.hs * kHeadDim; i += 256) {
    const int h = i >> 7, c = i & 127;
    const float L = hsum[h];
    qbuf[i] = L > 0.f ? (oacc[0][h][c] + oacc[1][h][c]) / L : 0.f;
    if (c == 0) lse2[h] = L > 0.f ? hm[h] + __log2f(L) : -INFINITY;
  }
  __syncthreads();
  write_result(a, u, qbuf, lse2);
}

// ---------------------------------------------------------------------------------------
// Attention over an unquantised fp32 K/V region: a window of recent tokens or a prefill kept
// unquantised ("RotaryQuant ...", method overview: deferred prefill; "RoPE-Aware Bit
// Allocation ...", results: the recent-token buffer).  fp16 regions take the matrix-core
// kernel (tq_dense.hip); fp32 values are not exact fp16 operands, so this one sums with fp32
// fused multiply-adds.  Same section split as the packed decode; each section's partial is
// rotated forward by R, so that it is in the rotated domain of the packed partials and the
// merge's one inverse rotation applies to both.
//
// One workgroup per (sequence, KV head, section, head slice of up to 8 heads), 64-token
// chunks: thread (token, quarter) forms 32-coordinate partial scores for every head, summed
// over the four quarter lanes by DPP; one wave per head runs the online softmax over the
// chunk; thread (8 coordinates, token slot) accumulates 4 tokens of each chunk per head.
// Raw 16-byte words of one thread's share of a 64-token chunk: 32 key values of its score
// token, 8 value coordinates of each of its 4 value tokens.
struct DenseRaw {
  static constexpr int KW = 8;  // 16-byte words per 32 values
  static constexpr int VW = 2;  // per 8 values
  uint4 k[KW];
  uint4 v[4][VW];
};

__device__ __forceinline__ void unpack8(const uint4* w, float* out) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    out[4 * j] = __uint_as_float(w[j].x);
    out[4 * j + 1] = __uint_as_float(w[j].y);
    out[4 * j + 2] = __uint_as_float(w[j].z);
    out[4 * j + 3] = __uint_as_float(w[j].w);
  }
}

template <bool QF16>
__global__ __launch_bounds__(256) void dense_kernel(const DenseArgs a) {
  constexpr int MAXH = 8;
  constexpr int ES = 4;  // bytes per value
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
  // lengths beyond max_len (checked against the capacity on the host) are clamped
  const int T = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_len)) : a.max_len;
  const int C = (T + a.n_splits - 1) / a.n_splits;
  const int lo = min(T, split * C), hi = min(T, lo + C);

  const size_t row0 = ((size_t)b * a.n_kv_heads + kv) * a.capacity;  // first token row of the stream
  const int st = tid >> 2, qd = tid & 3;                              // scores: token, quarter
  const int dg = tid & 15, ts = tid >> 4;                             // values: 8 coordinates, slot
  const uint8_t* kb = (const uint8_t*)a.k + row0 * kHeadDim * ES;
  const uint8_t* vb = (const uint8_t*)a.v + row0 * kHeadDim * ES;
  // this thread's raw words of the chunk at c0 (tokens past the section are not read)
  auto fetch = [&](int c0, DenseRaw& r) {
    const int tk = c0 + st;
    if (tk < hi) {
      const uint4* p = (const uint4*)(kb + ((size_t)tk * kHeadDim + 32 * qd) * ES);
#pragma unroll
      for (int i = 0; i < DenseRaw::KW; ++i) r.k[i] = p[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tv = c0 + ts + 16 * j;
      if (tv < hi) {
        const uint4* p = (const uint4*)(vb + ((size_t)tv * kHeadDim + 8 * dg) * ES);
#pragma unroll
        for (int i = 0; i < DenseRaw::VW; ++i) r.v[j][i] = p[i];
      }
    }
  };
  DenseRaw nxt;
  if (lo < hi) fetch(lo, nxt);  // the first chunk's reads overlap the query set-up

  for (int i = tid; i < hs * kHeadDim; i += 256) {
    const size_t qi = ((size_t)b * a.n_q_heads + h0 + (i >> 7)) * kHeadDim + (i & 127);
    qb[i] = (QF16 ? (float)((const _Float16*)a.q)[qi] : ((const float*)a.q)[qi]) * a.scale_log2;
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
    const DenseRaw cur = nxt;
    if (c0 + 64 < hi) fetch(c0 + 64, nxt);  // the next chunk loads during this one
    // scores of the chunk's tokens, all heads (scale and log2 e folded into the query)
    {
      const int tok = c0 + st;
      float kx[32];
#pragma unroll
      for (int i = 0; i < 4; ++i) unpack8(cur.k + 2 * i, kx + 8 * i);
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
    // value sums: tokens ts, ts + 16, ts + 32, ts + 48 of the chunk, coordinates 8dg .. +7
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
        if (c0 + ts + 16 * j < hi) {
          float vx[8];
          unpack8(cur.v[j], vx);
#pragma unroll
          for (int h = 0; h < MAXH; ++h) {
            if (h < hs) {
              const float p = pw[h][ts + 16 * j];
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
  // into the rotated domain of the packed partials: signs, normalised Hadamard, SO(4)
  lds_rotate<true>(qb, hs, a.signs + kv * kHeadDim, a.so4 ? a.so4 + kv * 256 : nullptr, a.rot_group);
  const size_t prow = ((size_t)split * a.batch + b) * a.n_q_heads + h0;
  if (tid < hs) a.part_lse[prow + tid] = lse2[tid] * kLn2;
  for (int i = tid; i < hs * kHeadDim; i += 256) a.part_o[(prow + (i >> 7)) * kHeadDim + (i & 127)] = qb[i];
}

// ---------------------------------------------------------------------------------------
// Log-sum-exp merge of key-axis splits plus the single inverse rotation.
// Inverse of query_rotate for one head held by 32 lanes (4 coordinates each): SO(4)
// inverse, the (self-inverse) normalised Hadamard, then the sign flips.
template <int GROUP>
__device__ __forceinline__ float4 unrotate4(float4 x, const QueryLane& s, bool so4, int lane) {
  Quat v{x.x, x.y, x.z, x.w};
  if (so4) v = qmul(qmul(qconj(s.l), v), s.r);
  float x0 = v.w, x1 = v.x, x2 = v.y, x3 = v.z;
  float y0 = x0 + x1, y1 = x0 - x1, y2 = x2 + x3, y3 = x2 - x3;
  x0 = y0 + y2; x1 = y1 + y3; x2 = y0 - y2; x3 = y1 - y3;
#pragma unroll
  for (int m = 1; m < GROUP / 4; m <<= 1) {
    const bool up = (lane & m) != 0;
    const float o0 = lane_xor(x0, m, lane), o1 = lane_xor(x1, m, lane), o2 = lane_xor(x2, m, lane),
                o3 = lane_xor(x3, m, lane);
    x0 = up ? o0 - x0 : x0 + o0;
    x1 = up ? o1 - x1 : x1 + o1;
    x2 = up ? o2 - x2 : x2 + o2;
    x3 = up ? o3 - x3 : x3 + o3;
  }
  const float hsc = GROUP == 32 ? 0.17677669529663688f : 0.088388347648318440f;
  return make_float4(x0 * hsc * s.sg.x, x1 * hsc * s.sg.y, x2 * hsc * s.sg.z, x3 * hsc * s.sg.w);
}

// Log-sum-exp merge of the split partials of one (sequence, query head) and the single
// inverse rotation.  Every global read that does not depend on another is issued first:
// the section lse values, the first partials, the signs and SO(4) parameters.  With many
// sections the workgroup has NP groups of 128 threads, group p taking sections p, p + NP,
// ..., so that the partials of up to 16 NP sections are in flight in one round trip; the NP
// sums meet in LDS.
template <int GROUP, int NP>
__global__ __launch_bounds__(128 * NP) void merge_kernel(const MergeArgs a) {
  constexpr int kMaxStage = 1024;
  constexpr int kAhead = 16;  // partials held in registers ahead of the weights
  constexpr int NT = 128 * NP, NWV = 2 * NP;
  __shared__ __attribute__((aligned(16))) float obuf[kHeadDim];
  __shared__ float psum[NP][kHeadDim];
  __shared__ float wts[kMaxStage];
  __shared__ float red[2][NWV];
  const int row = blockIdx.x;  // b * n_q_heads + h
  const int h = row % a.n_q_heads;
  const int kv = h / a.group_size;
  const int t = threadIdx.x, c = t & 127, p = t >> 7, lane = t & 63, wv = t >> 6;
  const size_t stride = (size_t)a.batch * a.n_q_heads;
  const int S = a.n_splits;
  const float* po = a.part_o + (size_t)row * kHeadDim + c;

  float lse0 = t < S ? a.part_lse[t * stride + row] : -INFINITY;
  float ahead[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) ahead[j] = p + NP * j < S ? po[(p + NP * j) * stride * kHeadDim] : 0.f;
  QueryLane rl;
  rl.live = wv == 0 && lane < 32;
  rl.sg = make_float4(1.f, 1.f, 1.f, 1.f);
  rl.l = rl.r = Quat{1.f, 0.f, 0.f, 0.f};
  if (rl.live && a.signs) {
    rl.sg = *(const float4*)(a.signs + kv * kHeadDim + 4 * lane);
    if (a.so4) {
      rl.l = qload(a.so4 + kv * 256 + 8 * lane);
      rl.r = qload(a.so4 + kv * 256 + 8 * lane + 4);
    }
  }

  // maximum lse, then the weights e^{lse_s - max} (in LDS when they fit) and their sum
  float M = lse0;
  for (int s = t + NT; s < S; s += NT) M = fmaxf(M, a.part_lse[s * stride + row]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[0][wv] = M;
  __syncthreads();
  M = red[0][0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) M = fmaxf(M, red[0][w]);
  const float mu = M == -INFINITY ? 0.f : M;
  float W = 0.f;
  for (int s = t; s < S; s += NT) {
    const float l = s == t ? lse0 : a.part_lse[s * stride + row];
    const float w = l == -INFINITY ? 0.f : expf(l - mu);
    if (s < kMaxStage) wts[s] = w;
    W += w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) W += __shfl_xor(W, o);
  if (lane == 0) red[1][wv] = W;
  __syncthreads();
  W = red[1][0];
#pragma unroll
  for (int w = 1; w < NWV; ++w) W += red[1][w];

  // weighted sum of this group's partials
  float acc = 0.f;
#pragma unroll
  for (int j = 0; j < kAhead; ++j)
    if (p + NP * j < S) acc = fmaf(wts[p + NP * j], ahead[j], acc);
  int s = p + NP * kAhead;
  for (; s + NP * 7 < S && s + NP * 7 < kMaxStage; s += NP * 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = po[(s + NP * j) * stride * kHeadDim];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = fmaf(wts[s + NP * j], v[j], acc);
  }
  for (; s < S; s += NP) {
    const float l = a.part_lse[s * stride + row];
    const float w = s < kMaxStage ? wts[s] : (l == -INFINITY ? 0.f : expf(l - mu));
    acc = fmaf(w, po[s * stride * kHeadDim], acc);
  }
  if (NP > 1) {
    psum[p][c] = acc;
    __syncthreads();
    if (p == 0) {
#pragma unroll
      for (int q = 1; q < NP; ++q) acc += psum[q][c];
    }
  }
  if (p == 0) obuf[c] = W > 0.f ? acc / W : 0.f;
  __syncthreads();
  if (wv == 0) {  // the whole first wave takes part in the lane exchanges
    const float4 x = *(const float4*)(obuf + 4 * (lane & 31));
    // partials formed in the original domain (no rotation given) are already the output
    const float4 y = a.signs ? unrotate4<GROUP>(x, rl, a.so4 != nullptr, lane) : x;
    if (rl.live) *(float4*)(a.out + (size_t)row * kHeadDim + 4 * lane) = y;
  }
  if (a.lse_out && t == 0) a.lse_out[row] = W > 0.f ? mu + logf(W) : -INFINITY;
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Launchers.

static int device_cus();

// Whole tiles go to the matrix-core append when the vectors are fp16, every row starts at
// the same position and at least one tile is whole: tiles [j0, j0 + n_full), counted from
// slot 0.  The partial tiles at either end (at most two per row) stay with the tile kernel,
// in its edge mode (tiles counted from pos0 / 32).  Calls of more than 2^22 vectors per row
// (a row's input past 1 GiB, beyond the kernel's 32-bit buffer offsets with room to spare)
// take the tile kernel whole.
static bool mfma_append_split(const AppendArgs& a, bool x_f16, int& j0, int& n_full, AppendArgs& edges) {
  if (!x_f16 || a.pos != nullptr || a.n_new < 2 * kTile || a.n_new > (1 << 22) || a.n_edges != 0) return false;
  const int first = (a.pos0 + kTile - 1) / kTile, end = (a.pos0 + a.n_new) / kTile;
  if (end <= first) return false;
  j0 = first;
  n_full = end - first;
  edges = a;
  edges.n_edges = 0;
  if (a.pos0 % kTile) edges.edge[edges.n_edges++] = 0;
  if ((a.pos0 + a.n_new) % kTile) edges.edge[edges.n_edges++] = end - a.pos0 / kTile;
  return true;
}

// Whole tiles per workgroup: one round of workgroups (per_cu per CU) over all rows (and
// roles), each wave with at least two tiles where there are enough.
static int mfma_append_chunks(int n_full, int rows, int per_cu, int& per_wg) {
  int chunks = std::max(1, std::min(n_full, (per_cu * device_cus() + rows - 1) / rows));
  per_wg = (n_full + chunks - 1) / chunks;
  return (n_full + per_wg - 1) / per_wg;
}

hipError_t launch_append(const AppendArgs& a, int bits, int group, bool values, bool x_f16, int batch,
                         int n_tiles, hipStream_t stream) {
  int j0 = 0, n_full = 0;
  AppendArgs edges;
  if (mfma_append_split(a, x_f16, j0, n_full, edges)) {
    int per_wg = 0;
    const dim3 mgrid(mfma_append_chunks(n_full, batch * a.n_kv_heads, group == 128 ? 2 : 3, per_wg), a.n_kv_heads,
                     batch);
    const bool ex = a.so4 == nullptr;  // a rotation without SO(4) blocks: exact +-1 operands
#define TQ_APPEND_M(B, G, V, E)                                                                          \
  if (bits == B && group == G && values == V && ex == E)                                                 \
    hipLaunchKernelGGL((append_mfma_kernel<B, G, V, E>), mgrid, dim3(64 * MfmaAppendShape<G>::kWaves), 0, stream, a, j0, \
                       n_full, per_wg);
#define TQ_APPEND_M2(B, G, V) TQ_APPEND_M(B, G, V, false) TQ_APPEND_M(B, G, V, true)
    TQ_APPEND_M2(3, 32, false) TQ_APPEND_M2(3, 32, true) TQ_APPEND_M2(3, 128, false) TQ_APPEND_M2(3, 128, true)
    TQ_APPEND_M2(4, 32, false) TQ_APPEND_M2(4, 32, true) TQ_APPEND_M2(4, 128, false) TQ_APPEND_M2(4, 128, true)
#undef TQ_APPEND_M2
#undef TQ_APPEND_M
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || edges.n_edges == 0) return e;
    return launch_append(edges, bits, group, values, x_f16, batch, edges.n_edges, stream);  // edge mode
  }
  const dim3 grid(n_tiles, a.n_kv_heads, batch), block(128);
#define TQ_APPEND(B, G, V, X)                                                        \
  if (bits == B && group == G && values == V && x_f16 == X) {                        \
    hipLaunchKernelGGL((append_kernel<B, G, V, X>), grid, block, 0, stream, a);      \
    return hipGetLastError();                                                        \
  }
#define TQ_APPEND_X(B, G, V) TQ_APPEND(B, G, V, true) TQ_APPEND(B, G, V, false)
#define TQ_APPEND_V(B, G) TQ_APPEND_X(B, G, true) TQ_APPEND_X(B, G, false)
  TQ_APPEND_V(3, 32) TQ_APPEND_V(3, 128) TQ_APPEND_V(4, 32) TQ_APPEND_V(4, 128)
#undef TQ_APPEND_V
#undef TQ_APPEND_X
#undef TQ_APPEND
  return hipErrorInvalidValue;
}

hipError_t launch_append_kv(const AppendArgs& ak, const AppendArgs& av, int bits_k, int bits_v, int group, bool x_f16,
                            int batch, int n_tiles, hipStream_t stream) {
  if (ak.n_new == 1) {
    const dim3 grid((batch * ak.n_kv_heads + 3) / 4), block(256);
#define TQ_STEP(BK, BV, G, X)                                                                    \
  if (bits_k == BK && bits_v == BV && group == G && x_f16 == X) {                                \
    hipLaunchKernelGGL((append_step_kernel<BK, BV, G, X>), grid, block, 0, stream, ak, av, batch); \
    return hipGetLastError();                                                                    \
  }
#define TQ_STEP_X(BK, BV, G) TQ_STEP(BK, BV, G, true) TQ_STEP(BK, BV, G, false)
#define TQ_STEP_G(BK, BV) TQ_STEP_X(BK, BV, 32) TQ_STEP_X(BK, BV, 128)
    TQ_STEP_G(3, 3) TQ_STEP_G(4, 3) TQ_STEP_G(3, 4) TQ_STEP_G(4, 4)
#undef TQ_STEP_G
#undef TQ_STEP_X
#undef TQ_STEP
    return hipErrorInvalidValue;
  }
  int j0 = 0, n_full = 0;
  AppendArgs ek, ev;
  if (mfma_append_split(ak, x_f16, j0, n_full, ek) && mfma_append_split(av, x_f16, j0, n_full, ev)) {
    int per_wg = 0;
    const dim3 mgrid(mfma_append_chunks(n_full, 2 * batch * ak.n_kv_heads, group == 128 ? 2 : 3, per_wg), ak.n_kv_heads,
                     2 * batch);
    const bool ex = ak.so4 == nullptr;  // a rotation without SO(4) blocks: exact +-1 operands
#define TQ_APPEND_KV_M(BK, BV, G, E)                                                                              \
  if (bits_k == BK && bits_v == BV && group == G && ex == E)                                                     \
    hipLaunchKernelGGL((append_mfma_kv_kernel<BK, BV, G, E>), mgrid, dim3(64 * MfmaAppendShape<G>::kWaves), 0, stream, ak, \
                       av, batch, j0, n_full, per_wg);
#define TQ_APPEND_KV_M2(BK, BV, G) TQ_APPEND_KV_M(BK, BV, G, false) TQ_APPEND_KV_M(BK, BV, G, true)
    TQ_APPEND_KV_M2(3, 3, 32) TQ_APPEND_KV_M2(3, 3, 128) TQ_APPEND_KV_M2(4, 3, 32) TQ_APPEND_KV_M2(4, 3, 128)
    TQ_APPEND_KV_M2(3, 4, 32) TQ_APPEND_KV_M2(3, 4, 128) TQ_APPEND_KV_M2(4, 4, 32) TQ_APPEND_KV_M2(4, 4, 128)
#undef TQ_APPEND_KV_M2
#undef TQ_APPEND_KV_M
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || ek.n_edges == 0) return e;
    return launch_append_kv(ek, ev, bits_k, bits_v, group, x_f16, batch, ek.n_edges, stream);  // edge mode
  }
  const dim3 grid(n_tiles, ak.n_kv_heads, 2 * batch), block(128);
#define TQ_APPEND_KV(BK, BV, G, X)                                                              \
  if (bits_k == BK && bits_v == BV && group == G && x_f16 == X) {                              \
    hipLaunchKernelGGL((append_kv_kernel<BK, BV, G, X>), grid, block, 0, stream, ak, av, batch); \
    return hipGetLastError();                                                                  \
  }
#define TQ_APPEND_KV_X(BK, BV, G) TQ_APPEND_KV(BK, BV, G, true) TQ_APPEND_KV(BK, BV, G, false)
#define TQ_APPEND_KV_G(BK, BV) TQ_APPEND_KV_X(BK, BV, 32) TQ_APPEND_KV_X(BK, BV, 128)
  TQ_APPEND_KV_G(3, 3) TQ_APPEND_KV_G(4, 3) TQ_APPEND_KV_G(3, 4) TQ_APPEND_KV_G(4, 4)
#undef TQ_APPEND_KV_G
#undef TQ_APPEND_KV_X
#undef TQ_APPEND_KV
  return hipErrorInvalidValue;
}

// The section partials of the allocation-free decode step live here, one copy per device,
// for callers that cannot allocate (HIP graph capture, serving loops).  In host code the
// array's name is not a device address: every host use goes through the address
// hipGetSymbolAddress returns for the current device, looked up once per device and kept.
static __device__ __align__(256) float scratch[kStaticPartialFloats];

hipError_t static_partials(float** p) {
  static std::atomic<float*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  float* a = addr[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    void* q = nullptr;
    if ((e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    a = (float*)q;
    addr[dev].store(a, std::memory_order_release);
  }
  *p = a;
  return hipSuccess;
}

// Compute units of the current device, read once per device.  The cache is atomic: calls
// from several host threads may both read the attribute and store the same value.
static int device_cus() {
  static std::atomic<int> cus[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

hipError_t launch_decode(const DecodeArgs& a, int schedule, int bits_k, int bits_v, bool q_f16, bool shared_table,
                         hipStream_t stream) {
  const int units = a.batch * a.n_kv_heads * a.n_splits * a.n_slices;
  const dim3 grid(units), block(256);
  const int ng = kHeadDim / a.rot_group;
  if (schedule == 2) {
    // a grid that leaves CUs without a second workgroup runs eight waves per workgroup
    const int nw = units <= device_cus() ? 8 : 4;
    // blocks per wave (an upper bound): a one-block ring where a wave holds fewer than four
    const int per_wave = ((a.max_len + a.n_splits - 1) / a.n_splits + 2 * kTile - 1) / kTile / nw;
    const bool deep = ng == 1 || per_wave >= 4;
#define TQ_MF_D(BK, BV, NG, QF, QD, NW)                                                                  \
  if (deep)                                                                                             \
    hipLaunchKernelGGL((decode_mfma_kernel<BK, BV, NG, QF, QD, NW, 2>), grid, dim3(64 * NW), 0, stream, a); \
  else                                                                                                  \
    hipLaunchKernelGGL((decode_mfma_kernel<BK, BV, NG, QF, QD, NW, NG == 1 ? 2 : 1>), grid, dim3(64 * NW), 0, stream, a);
#define TQ_MF(BK, BV, NG, QF, QD)                                                        \
  if (bits_k == BK && bits_v == BV && ng == NG && q_f16 == QF && shared_table == QD) {    \
    if (nw == 8) {                                                                       \
      TQ_MF_D(BK, BV, NG, QF, QD, 8)                                                     \
    } else {                                                                             \
      TQ_MF_D(BK, BV, NG, QF, QD, 4)                                                     \
    }                                                                                    \
    return hipGetLastError();                                                            \
  }
#define TQ_MF_Q(BK, BV, NG, QD) TQ_MF(BK, BV, NG, true, QD) TQ_MF(BK, BV, NG, false, QD)
#define TQ_MF_NG(BK, BV, QD) TQ_MF_Q(BK, BV, 4, QD) TQ_MF_Q(BK, BV, 1, QD)
    TQ_MF_NG(3, 3, true) TQ_MF_NG(3, 3, false) TQ_MF_NG(4, 4, false) TQ_MF_NG(4, 3, false) TQ_MF_NG(3, 4, false)
#undef TQ_MF_NG
#undef TQ_MF_Q
#undef TQ_MF
#undef TQ_MF_D
  } else {
#define TQ_VEC(BK, BV, NG, QF)                                                               \
  if (bits_k == BK && bits_v == BV && ng == NG && q_f16 == QF) {                             \
    hipLaunchKernelGGL((decode_vec_kernel<BK, BV, NG, QF>), grid, block, 0, stream, a);      \
    return hipGetLastError();                                                                \
  }
#define TQ_VEC_Q(BK, BV, NG) TQ_VEC(BK, BV, NG, true) TQ_VEC(BK, BV, NG, false)
#define TQ_VEC_NG(BK, BV) TQ_VEC_Q(BK, BV, 4) TQ_VEC_Q(BK, BV, 1)
    TQ_VEC_NG(3, 3) TQ_VEC_NG(4, 4) TQ_VEC_NG(4, 3) TQ_VEC_NG(3, 4)
#undef TQ_VEC_NG
#undef TQ_VEC_Q
#undef TQ_VEC
  }
  return hipErrorInvalidValue;
}

hipError_t launch_dense(const DenseArgs& a, bool kv_f16, bool q_f16, hipStream_t stream) {
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(256);
  if (kv_f16) return launch_dense_mfma(a, q_f16, stream);  // fp16 rows are exact matrix-core operands
  if (q_f16) hipLaunchKernelGGL((dense_kernel<true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((dense_kernel<false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  // sections per 128-thread group: the first 16 of each group are read in one round trip
  const int np = a.n_splits > 32 ? 4 : a.n_splits > 16 ? 2 : 1;
  const dim3 grid(a.batch * a.n_q_heads), block(128 * np);
#define TQ_MERGE(G, NP) \
  if (a.rot_group == G && np == NP) hipLaunchKernelGGL((merge_kernel<G, NP>), grid, block, 0, stream, a);
  TQ_MERGE(32, 1) TQ_MERGE(32, 2) TQ_MERGE(32, 4) TQ_MERGE(128, 1) TQ_MERGE(128, 2) TQ_MERGE(128, 4)
#undef TQ_MERGE
  return hipGetLastError();
}

}  // namespace tq

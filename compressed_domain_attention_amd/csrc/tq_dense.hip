// Decode attention over an unquantised fp16 K/V region on the matrix cores, written as key-axis
// section partials in the packed cache's rotated domain.  Target: gfx950 (MI355X), wave64.
//
// Method source: "RotaryQuant ... Fused Compressed-Space Attention", method overview (the
// prefill is kept in fp16 and quantised later) and "RoPE-Aware Bit Allocation for KV-Cache
// Quantization", results and limitations (a recent-token buffer in full precision): decode
// attention reads those tokens as they are, and its partials merge with the packed cache's.
//
// One workgroup of NW waves per (sequence, KV head, section, slice of up to 8 query heads).
// The section's 16-token tiles go to the waves in turn; each wave streams its tiles through
// its own ring of D LDS stages filled by direct global -> LDS copies (a stage: 16 key rows
// and 16 value rows of 256 bytes).  Key rows are exact fp16 operands: the score product is
// v_mfma_f32_16x16x32_f16 with the key row of token col as the A row against the query's
// fp16 high (columns 0-7) and low (8-15) parts, so scores keep fp32-level accuracy.  Key rows
// land swizzled (16-byte chunk c of row r at chunk c ^ r of the row), so that the sixteen
// rows read at one chunk index fall in different banks.  The lazy softmax reference, the
// 16x16x16 weight x value product (weights as fp16 high + low rows, values of four tokens
// paired by byte permutes) and the merge of the waves follow the Block-GTQ attention kernel.
// The merged output is rotated forward (signs, normalised Hadamard, SO(4)) into the packed
// partials' domain, so one merge with the single inverse rotation covers both stores.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2d = 0.69314718055994531f;
constexpr float kRescaleD = 8.f;  // log2 headroom of the lazily updated softmax reference

__device__ __forceinline__ f32x4 mfma_k32(u32x4 x, u32x4 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, x), __builtin_bit_cast(half8_t, y), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(u32x2 x, u32x2 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, x), __builtin_bit_cast(half4_t, y), c, 0, 0,
                                               0);
}
__device__ __forceinline__ uint32_t pack2(float x, float y) {
  return __builtin_bit_cast(uint32_t, half2_t{(_Float16)x, (_Float16)y});
}
__device__ __forceinline__ float lo_part(float x) { return x - (float)(_Float16)x; }
template <typename T>
__device__ __forceinline__ T lds_ld(const uint8_t* p) {
  return *(const T*)p;
}

template <int NW, int D, bool QF16>
__global__ __launch_bounds__(64 * NW) void dense_mfma_kernel(const DenseArgs a) {
  constexpr int VAL_AT = 4096, STAGE = 8192;  // key rows 4 KB (swizzled), value rows 4 KB
  constexpr int NDMA = 8;                     // 16-byte copies per lane and stage
  constexpr int WAVE_LDS = D * STAGE;
  static_assert(D >= 2 && D * NDMA <= 63, "ring depth within the memory counter");
  __shared__ __attribute__((aligned(16))) uint8_t lds[NW * WAVE_LDS];
  __shared__ __attribute__((aligned(16))) float qraw[8][128];  // scaled query rows, later the output
  __shared__ float part_m[NW][8], part_l[NW][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / a.n_slices, slice = blockIdx.x - unit * a.n_slices;
  const int split = unit % a.n_splits, kv = (unit / a.n_splits) % a.n_kv_heads;
  const int b = unit / (a.n_splits * a.n_kv_heads);
  const int h0 = kv * a.group_size + slice * a.heads_per_slice;
  const int hs = min(a.heads_per_slice, a.group_size - slice * a.heads_per_slice);
  // lengths beyond max_len (checked against the capacity on the host) are clamped
  const int T = a.seq_lens ? max(0, min(a.seq_lens[b], a.max_len)) : a.max_len;
  const int C = (T + a.n_splits - 1) / a.n_splits;
  const int lo = min(T, split * C), hi = min(T, lo + C);
  const int ntiles = lo < hi ? (hi - lo + 15) >> 4 : 0;
  const int n = ntiles > wv ? (ntiles - wv + NW - 1) / NW : 0;  // this wave's tiles

  const size_t row0 = ((size_t)b * a.n_kv_heads + kv) * a.capacity;
  const uint8_t* kbase = (const uint8_t*)a.k + row0 * 256;
  const uint8_t* vbase = (const uint8_t*)a.v + row0 * 256;
  const int cap = a.capacity;
  uint8_t* wlds = lds + wv * WAVE_LDS;
  const uint32_t wlds_a = lds_addr(wlds);
  auto tok0_of = [&](int s) { return lo + 16 * (wv + NW * s); };
  // stage s: copy k moves rows 4k .. 4k + 3; key chunk index 16 r + j holds the row's
  // chunk j ^ r; rows past the capacity are replaced by the tile's first (weights 0)
  auto issue = [&](int s) {
    const int t0 = tok0_of(s);
    const uint32_t dst = wlds_a + (s % D) * STAGE;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 4 * k + (lane >> 4), j = lane & 15, t = t0 + r;
      lds_dma<16, true>(dst + 1024 * k, kbase, t < cap ? (uint32_t)t * 256u + 16u * (j ^ r) : (uint32_t)t0 * 256u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int t = t0 + 4 * k + (lane >> 4);
      lds_dma<16, true>(dst + VAL_AT + 1024 * k, vbase,
                        t < cap ? (uint32_t)t * 256u + 16u * (lane & 15) : (uint32_t)t0 * 256u);
    }
  };

  // the slice's query rows, scaled (log2 units); heads past the slice are zero
  for (int i = tid; i < 8 * 128; i += 64 * NW) {
    const int hh = i >> 7, c = i & 127;
    const size_t qi = ((size_t)b * a.n_q_heads + h0 + hh) * 128 + c;
    qraw[hh][c] = hh >= hs ? 0.f : (QF16 ? (float)((const _Float16*)a.q)[qi] : ((const float*)a.q)[qi]) * a.scale_log2;
  }
  __syncthreads();
  const int col = lane & 15, jr = lane >> 4;
  // query operands of k-step ks: coordinates 32 ks + 8 jr .. + 7 of head col & 7, fp16 high
  // parts in columns 0-7 and low parts in 8-15
  u32x4 qk[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint32_t x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v0 = qraw[col & 7][32 * ks + 8 * jr + 2 * e], v1 = qraw[col & 7][32 * ks + 8 * jr + 2 * e + 1];
      x[e] = col >= 8 ? pack2(lo_part(v0), lo_part(v1)) : pack2(v0, v1);
    }
    qk[ks] = u32x4{x[0], x[1], x[2], x[3]};
  }
  for (int s = 0; s < D; ++s)
    if (s < n) issue(s);

  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, thr = -INFINITY, lsum = 0.f;

  for (int s = 0; s < n; ++s) {
    if (min(D - 1, n - 1 - s) >= 1) vm_wait<NDMA>();
    else vm_wait<0>();
    const int t0 = tok0_of(s);
    const int nv = min(16, hi - t0);
    const uint8_t* sb = wlds + (s % D) * STAGE;

    // ---- scores: the key operand row is token col, its k slots coordinates 32 ks + 8 jr ..
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      sc = mfma_k32(lds_ld<u32x4>(sb + 16 * (16 * col + ((4 * ks + jr) ^ col))), qk[ks], sc);
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = sc[e] + dpp<0x128>(sc[e]);  // high + low query parts
      x[e] = 4 * jr + e < nv ? v : -INFINITY;
      bm = fmaxf(bm, x[e]);
    }
    bm = max_rows(bm);
    if (__builtin_expect(__builtin_amdgcn_ballot_w64(bm > thr) != 0, 0)) {
      const float mnew = fmaxf(mref, bm);
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float al = __shfl(alpha, (4 * jr + e) & 7);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc[ct][e] *= al;
      }
      mref = mnew;
      thr = mnew + kRescaleD;
    }
    u32x2 pf;
    {
      float pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = __builtin_amdgcn_exp2f(x[e] - mref);
        lsum += pw[e];
        if (col >= 8) pw[e] = lo_part(pw[e]);
      }
      pf = u32x2{pack2(pw[0], pw[1]), pack2(pw[2], pw[3])};
    }
    // ---- output: values of tokens 4 jr .. + 3; tile ct holds coordinate
    // 64 (ct / 4) + 4 col + ct % 4, so one 8-byte read per token serves four tiles
    u32x2 vw[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint2 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = lds_ld<uint2>(sb + VAL_AT + 256 * (4 * jr + e) + 128 * u + 8 * col);
      vw[4 * u + 0] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, 0x05040100u), __builtin_amdgcn_perm(r[3].x, r[2].x, 0x05040100u)};
      vw[4 * u + 1] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, 0x07060302u), __builtin_amdgcn_perm(r[3].x, r[2].x, 0x07060302u)};
      vw[4 * u + 2] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, 0x05040100u), __builtin_amdgcn_perm(r[3].y, r[2].y, 0x05040100u)};
      vw[4 * u + 3] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, 0x07060302u), __builtin_amdgcn_perm(r[3].y, r[2].y, 0x07060302u)};
    }
    if (nv < 16) {  // a partial tile: tokens past the section carry zeros (their weights are 0)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int t = 4 * jr;
        vw[ct].x &= (t < nv ? 0xFFFFu : 0u) | (t + 1 < nv ? 0xFFFF0000u : 0u);
        vw[ct].y &= (t + 2 < nv ? 0xFFFFu : 0u) | (t + 3 < nv ? 0xFFFF0000u : 0u);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = mfma_k16(pf, vw[ct], acc[ct]);
    if (s + D < n) {
      lds_wait();
      issue(s + D);
    }
  }

  // ---- merge the waves, normalise, rotate into the packed partials' domain
  vm_wait<0>();
  lsum = sum_rows(lsum);
  __syncthreads();
  float* po = (float*)wlds;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float o0, o1;
      pair32(acc[ct][e], o0, o1);
      if (jr < 2) po[(4 * jr + e) * 128 + 64 * (ct >> 2) + 4 * col + (ct & 3)] = o0 + o1;
    }
  if (lane < 8) {
    part_m[wv][lane] = mref;
    part_l[wv][lane] = lsum;
  }
  __syncthreads();
  for (int idx = tid; idx < hs * 128; idx += 64 * NW) {
    const int h = idx >> 7, c = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, part_m[w][h]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = part_m[w][h] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(part_m[w][h] - M);
      L += f * part_l[w][h];
      O += f * ((const float*)(lds + w * WAVE_LDS))[h * 128 + c];
    }
    qraw[h][c] = L > 0.f ? O / L : 0.f;
    if (c == 0) {
      const size_t prow = ((size_t)split * a.batch + b) * a.n_q_heads + h0 + h;
      a.part_lse[prow] = L > 0.f ? (M + __log2f(L)) * kLn2d : -INFINITY;
    }
  }
  __syncthreads();
  lds_rotate<true>(&qraw[0][0], hs, a.signs + kv * 128, a.so4 ? a.so4 + kv * 256 : nullptr, a.rot_group);
  const size_t prow = ((size_t)split * a.batch + b) * a.n_q_heads + h0;
  for (int i = tid; i < hs * 128; i += 64 * NW) a.part_o[(prow + (i >> 7)) * 128 + (i & 127)] = qraw[i >> 7][i & 127];
}

}  // namespace

hipError_t launch_dense_mfma(const DenseArgs& a, bool q_f16, hipStream_t stream) {
  constexpr int NW = 4, D = 2;
  if (a.heads_per_slice > 8) return hipErrorInvalidValue;
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(64 * NW);
  if (q_f16) hipLaunchKernelGGL((dense_mfma_kernel<NW, D, true>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((dense_mfma_kernel<NW, D, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace tq

// HIP kernels for Block-GTQ keys: encoding keys with one TQ-MSE encoder per bit width, and
// decode attention over those keys with fp16 values.  Target: gfx950 (MI355X), wave64.
//
// Method source: "RoPE-Aware Bit Allocation for KV-Cache Quantization" (aitrends.kr):
// blocks of equal width share one TQ-MSE encoder (norm -> normalise -> random rotation ->
// Lloyd-Max search); the logit q . k is an exact sum over the groups, so with the query
// rotated by each group's rotation (q~_g = Q_g^T q_g) a key's score is
// sum_g norm_g sum_{j in g} q~_j c_g[code_j]; values stay in fp16 (the page's keys-only
// evaluation).  Key records and the encoder layout are described in tq.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tq.h"
#include "tq_internal.h"
#include "tq_device.h"

namespace tq {
namespace {

constexpr float kLn2g = 0.69314718055994531f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x += __shfl_xor(x, o);
  return x;
}

// Group of group-order position j: the number of later groups' starts it has passed.
__device__ __forceinline__ int group_of(const tq_gtq_head& h, int j) {
  return (j >= h.start[1]) + (j >= h.start[2]) + (j >= h.start[3]);
}

// Copies one head's encoder into LDS (all threads of the block take part).
__device__ __forceinline__ void stage_head(tq_gtq_head* dst, const tq_gtq_head* src) {
  constexpr int words = sizeof(tq_gtq_head) / 4;
  for (int i = threadIdx.x; i < words; i += blockDim.x) ((uint32_t*)dst)[i] = ((const uint32_t*)src)[i];
}

// ---------------------------------------------------------------------------------------
// Key encoding.  One workgroup per (64-token tile, KV head, sequence) stages the head's
// encoder and rotations in LDS; each wave encodes one token at a time: lane l holds
// group-order positions 2l and 2l + 1 (always in one group: groups start at even positions
// and have even sizes).
template <bool XF16>
__global__ __launch_bounds__(256) void gtq_quantize_kernel(const GtqQuantArgs a) {
  __shared__ float rot[TQ_GTQ_ROTATION_FLOATS];
  __shared__ float ubuf[4][128];
  __shared__ tq_gtq_head hd;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  stage_head(&hd, (const tq_gtq_head*)a.heads + h);
  __syncthreads();
  int used = 0;
  for (int g = 0; g < hd.n_groups; ++g) used = hd.rot_offset[g] + hd.dim[g] * hd.dim[g];
  const float* grot = a.rotations + (size_t)h * TQ_GTQ_ROTATION_FLOATS;
  for (int i = tid; i < used; i += 256) rot[i] = grot[i];
  __syncthreads();

  const int j0 = 2 * lane;
  const int g = group_of(hd, j0);
  const int st = hd.start[g], n = hd.dim[g], off = hd.rot_offset[g];
  const int nb = (1 << hd.width[g]) - 1;
  const size_t stream = (size_t)b * a.n_kv_heads + h;
  for (int t = wv; t < 64; t += 4) {
    const int i = tile * 64 + t;
    if (i >= a.n_new) break;
    const size_t xrow = (stream * a.n_new + i) * 128;
    float x0, x1;
    if (XF16) {
      x0 = (float)((const _Float16*)a.x)[xrow + hd.coord[j0]];
      x1 = (float)((const _Float16*)a.x)[xrow + hd.coord[j0 + 1]];
    } else {
      x0 = ((const float*)a.x)[xrow + hd.coord[j0]];
      x1 = ((const float*)a.x)[xrow + hd.coord[j0 + 1]];
    }
    const float sq = x0 * x0 + x1 * x1;
    float ss[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) ss[k] = wave_sum(g == k ? sq : 0.f);
    const float nu = sqrtf(g == 0 ? ss[0] : g == 1 ? ss[1] : g == 2 ? ss[2] : ss[3]);
    ubuf[wv][j0] = nu > 0.f ? x0 / nu : 0.f;
    ubuf[wv][j0 + 1] = nu > 0.f ? x1 / nu : 0.f;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // y = Q^T u for this lane's two positions of its group
    float y0 = 0.f, y1 = 0.f;
    const float* q0 = rot + off + (j0 - st);
    for (int r = 0; r < n; ++r) {
      const float u = ubuf[wv][st + r];
      y0 = fmaf(q0[r * n], u, y0);
      y1 = fmaf(q0[r * n + 1], u, y1);
    }
    uint32_t c0 = 0, c1 = 0;
    for (int k = 0; k < nb; ++k) {  // compare-count against the group's boundaries
      c0 += y0 > hd.boundary[g][k];
      c1 += y1 > hd.boundary[g][k];
    }
    const size_t rec = stream * a.capacity + a.pos0 + i;
    a.codes[rec * 64 + lane] = (uint8_t)(c0 | (c1 << 4));
    if (lane < 4) a.norms[rec * 4 + lane] = lane < hd.n_groups ? sqrtf(ss[lane & 3]) : 0.f;
    // the next token's writes to ubuf follow this token's reads in program order
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------------------
// Decode attention over Block-GTQ keys and fp16 values, vector arithmetic in fp32.  One
// workgroup per (sequence, KV head, section, head slice of up to 8 heads).  The prologue
// rotates the slice's queries by every group's rotation into group order (scale and log2 e
// folded in).  64-token chunks: thread (token, quarter) decodes the 32 group-order
// positions of its quarter (code -> the group's centroid -> times the group norm) and forms
// partial scores for every head, summed over the quarter lanes; one wave per head runs the
// online softmax over the chunk; thread (8 coordinates, token slot) adds 4 tokens of the
// chunk for every head.  Results are in the original domain.
template <int MAXH, bool QF16>
__global__ __launch_bounds__(256) void gtq_attention_kernel(const GtqAttnArgs a) {
  __shared__ __attribute__((aligned(16))) float qb[MAXH * 128];  // rotated query, later the output
  __shared__ float pw[MAXH][64];
  __shared__ float hm[MAXH], hsum[MAXH], halpha[MAXH];
  __shared__ __attribute__((aligned(16))) float ob[4][MAXH][128];
  __shared__ float lse2[MAXH];
  __shared__ float cbt[4][16];
  __shared__ tq_gtq_head hd;

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

  const size_t row0 = ((size_t)b * a.n_kv_heads + kv) * a.capacity;
  const int st = tid >> 2, qd = tid & 3;   // scores: token, quarter
  const int dg = tid & 15, ts = tid >> 4;  // values: 8 coordinates, token slot
  const uint8_t* kc = a.codes + row0 * 64;
  const float* kn = a.norms + row0 * 4;
  const uint8_t* vb = (const uint8_t*)a.v + row0 * 128 * 2;

  uint4 nk, nv[4];
  float4 nn;
  auto fetch = [&](int c0) {
    const int tk = c0 + st;
    if (tk < hi) {
      nk = *(const uint4*)(kc + (size_t)tk * 64 + 16 * qd);
      nn = *(const float4*)(kn + (size_t)tk * 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int tv = c0 + ts + 16 * j;
      if (tv < hi) nv[j] = *(const uint4*)(vb + ((size_t)tv * 128 + 8 * dg) * 2);
    }
  };
  if (lo < hi) fetch(lo);  // the first chunk's reads overlap the set-up

  stage_head(&hd, (const tq_gtq_head*)a.heads + kv);
  __syncthreads();
  if (tid < 64) cbt[tid >> 4][tid & 15] = hd.centroid[tid >> 4][tid & 15];
  {
    // q~_j = sum_r Q_g[r][j - start] q[coord[start + r]] for group-order position j
    const float* grot = a.rotations + (size_t)kv * TQ_GTQ_ROTATION_FLOATS;
    for (int i = tid; i < hs * 128; i += 256) {
      const int hh = i >> 7, j = i & 127;
      const int g = group_of(hd, j), s0 = hd.start[g], n = hd.dim[g];
      const size_t qbase = ((size_t)b * a.n_q_heads + h0 + hh) * 128;
      const float* rr = grot + hd.rot_offset[g] + (j - s0);
      float acc = 0.f;
      for (int r = 0; r < n; ++r) {
        const int c = hd.coord[s0 + r];
        const float x = QF16 ? (float)((const _Float16*)a.q)[qbase + c] : ((const float*)a.q)[qbase + c];
        acc = fmaf(rr[r * n], x, acc);
      }
      qb[i] = acc * a.scale_log2;
    }
  }
  if (tid < MAXH) {
    hm[tid] = -INFINITY;
    hsum[tid] = 0.f;
  }
  // this lane's 32 positions 32 qd + e: their groups, two bits each
  uint32_t gbits0 = 0, gbits1 = 0;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    gbits0 |= (uint32_t)group_of(hd, 32 * qd + e) << (2 * e);
    gbits1 |= (uint32_t)group_of(hd, 32 * qd + 16 + e) << (2 * e);
  }
  __syncthreads();

  float acc[MAXH][8];
#pragma unroll
  for (int h = 0; h < MAXH; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

  for (int c0 = lo; c0 < hi; c0 += 64) {
    const uint4 ck = nk;
    const float4 cn = nn;
    const uint4 cv0 = nv[0], cv1 = nv[1], cv2 = nv[2], cv3 = nv[3];
    if (c0 + 64 < hi) fetch(c0 + 64);
    // scores of the chunk's tokens, all heads
    {
      const int tok = c0 + st;
      const uint32_t w[4] = {ck.x, ck.y, ck.z, ck.w};
      float kx[32];
#pragma unroll
      for (int e = 0; e < 32; ++e) {
        const uint32_t code = (w[e >> 3] >> (4 * (e & 7))) & 15u;
        const uint32_t g = ((e < 16 ? gbits0 : gbits1) >> (2 * (e & 15))) & 3u;
        const float nu = g == 0 ? cn.x : g == 1 ? cn.y : g == 2 ? cn.z : cn.w;
        kx[e] = cbt[g][code] * nu;
      }
#pragma unroll
      for (int h = 0; h < MAXH; ++h) {
        if (h < hs) {
          const float4* qp = (const float4*)(qb + h * 128 + 32 * qd);
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
    // value sums: tokens ts, ts + 16, ts + 32, ts + 48 of the chunk, coordinates 8 dg .. + 7
    {
#pragma unroll
      for (int h = 0; h < MAXH; ++h) {
        if (h < hs) {
          const float al = halpha[h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= al;
        }
      }
      const uint4 cvs[4] = {cv0, cv1, cv2, cv3};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + ts + 16 * j < hi) {
          const uint32_t x[4] = {cvs[j].x, cvs[j].y, cvs[j].z, cvs[j].w};
          float vx[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
            const h2_t hh = __builtin_bit_cast(h2_t, x[e]);
            vx[2 * e] = (float)hh[0];
            vx[2 * e + 1] = (float)hh[1];
          }
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
  for (int i = tid; i < hs * 128; i += 256) {
    const int h = i >> 7, c = i & 127;
    const float L = hsum[h];
    qb[i] = L > 0.f ? (ob[0][h][c] + ob[1][h][c] + ob[2][h][c] + ob[3][h][c]) / L : 0.f;
    if (c == 0) lse2[h] = L > 0.f ? hm[h] + __log2f(L) : -INFINITY;
  }
  __syncthreads();
  if (a.n_splits == 1) {
    const size_t row = (size_t)b * a.n_q_heads + h0;
    if (a.lse_out && tid < hs) a.lse_out[row + tid] = lse2[tid] * kLn2g;
    for (int i = tid; i < hs * 128; i += 256) a.out[(row + (i >> 7)) * 128 + (i & 127)] = qb[i];
  } else {
    const size_t prow = ((size_t)split * a.batch + b) * a.n_q_heads + h0;
    if (tid < hs) a.part_lse[prow + tid] = lse2[tid] * kLn2g;
    for (int i = tid; i < hs * 128; i += 256) a.part_o[(prow + (i >> 7)) * 128 + (i & 127)] = qb[i];
  }
}

}  // namespace

hipError_t launch_gtq_quantize(const GtqQuantArgs& a, bool x_f16, int batch, hipStream_t stream) {
  const dim3 grid((a.n_new + 63) / 64, a.n_kv_heads, batch), block(256);
  if (x_f16) hipLaunchKernelGGL(gtq_quantize_kernel<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(gtq_quantize_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_gtq_attention(const GtqAttnArgs& a, bool q_f16, hipStream_t stream) {
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(256);
  // slices of up to 4 heads keep the accumulators of a thread at 32 registers
  if (a.heads_per_slice <= 4) {
    if (q_f16) hipLaunchKernelGGL((gtq_attention_kernel<4, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gtq_attention_kernel<4, false>), grid, block, 0, stream, a);
  } else {
    if (q_f16) hipLaunchKernelGGL((gtq_attention_kernel<8, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((gtq_attention_kernel<8, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace tq

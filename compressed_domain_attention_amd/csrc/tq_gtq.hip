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
#include <stddef.h>
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

template <typename T>
__device__ __forceinline__ T lds_read(const uint8_t* p) {
  return *(const T*)p;
}

// Copies one head's encoder into LDS (all threads of the block take part).
// bit k of x (k < 16) moves to bit 2k
__device__ __forceinline__ uint32_t spread_bits(uint32_t x) {
  x = (x | (x << 8)) & 0x00FF00FFu;
  x = (x | (x << 4)) & 0x0F0F0F0Fu;
  x = (x | (x << 2)) & 0x33333333u;
  return (x | (x << 1)) & 0x55555555u;
}

// Number of the sorted boundaries bnd[0 .. nb) strictly below y (the compare-count code), by
// binary search: at most 8 steps for the 255 boundaries of an 8-bit codebook.
__device__ __forceinline__ uint32_t count_below(float y, const float* bnd, int nb) {
  int lo = 0, hi = nb;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (bnd[mid] < y) lo = mid + 1;
    else hi = mid;
  }
  return (uint32_t)lo;
}

__device__ __forceinline__ void stage_head(tq_gtq_head* dst, const tq_gtq_head* src) {
  constexpr int words = sizeof(tq_gtq_head) / 4;
  for (int i = threadIdx.x; i < words; i += blockDim.x) ((uint32_t*)dst)[i] = ((const uint32_t*)src)[i];
}
// The same for a kernel whose codes never pass LEVELS levels: the layout fields, the first
// LEVELS centroids and LEVELS - 1 boundaries of every group and the fp16 scales (a quarter of
// a kilobyte of codebook instead of eight for nibble codes).
template <int LEVELS>
__device__ __forceinline__ void stage_head_part(tq_gtq_head* dst, const tq_gtq_head* src) {
  constexpr int pre = offsetof(tq_gtq_head, centroid) / 4, cen = pre;
  constexpr int bnd = offsetof(tq_gtq_head, boundary) / 4, fs = offsetof(tq_gtq_head, f16_scale) / 4;
  constexpr int G = TQ_GTQ_MAX_GROUPS, cw = LEVELS, bw = LEVELS - 1;
  constexpr int total = pre + G * cw + G * bw + G;
  for (int i = threadIdx.x; i < total; i += blockDim.x) {
    int w;
    if (i < pre) {
      w = i;
    } else if (i < pre + G * cw) {
      const int j = i - pre;
      w = cen + (j / cw) * 256 + j % cw;
    } else if (i < pre + G * cw + G * bw) {
      const int j = i - pre - G * cw;
      w = bnd + (j / bw) * 255 + j % bw;
    } else {
      w = fs + (i - pre - G * cw - G * bw);
    }
    ((uint32_t*)dst)[w] = ((const uint32_t*)src)[w];
  }
}

// Encodes one key x[128] (fp16 or fp32) into its record: group norms, the normalised group
// vector through the wave's 128 floats of LDS (ubuf), y = Q^T u for lane l's group-order
// positions 2l and 2l + 1 (always in one group: groups start at even positions and have
// even sizes), compare-count, one code byte per lane and one norm per group.  rot: the
// head's rotations, in LDS or global memory.  Every lane of the wave takes part.
// QJL (two-stage keys, one group): also the m = 128 sign bits of S r into sign_rec and
// sqrt(pi/2)/m |r| into norm slot 1, from the rotated-domain residual e = y - c_hat
// (S r = |x| M e with M = S Q; proj[j][i] = M[i][j], in LDS or global memory).
// PK (two-stage keys: the first stage's width, 1 to 3): the 128 codes are written
// bit-packed, code of position i at bit PK i of the record's little-endian bit string (16 PK
// bytes), and compared against the first 2^PK - 1 boundaries only, so every code fits its
// field whatever the head's width.  PK = 0: a Block-GTQ record of rec_bytes code bytes, a
// nibble per position of groups up to 4 bits and a byte per position of wider ones (at the
// head's byte_at), zeros from code_used on; nothing is written past rec_bytes.
template <bool XF16, bool QJL = false, int PK = 0>
__device__ __forceinline__ void encode_key(const tq_gtq_head& hd, const float* rot, const void* x, float* ubuf,
                                           uint8_t* code_rec, float* norm_rec, int lane, const float* proj = nullptr,
                                           uint8_t* sign_rec = nullptr, int rec_bytes = 64) {
  const int j0 = 2 * lane;
  const int g = group_of(hd, j0);
  const int st = hd.start[g], n = hd.dim[g], off = hd.rot_offset[g];
  const int nb = PK ? min((1 << hd.width[g]) - 1, (1 << PK) - 1) : (1 << hd.width[g]) - 1;
  float x0, x1;
  if (XF16) {
    x0 = (float)((const _Float16*)x)[hd.coord[j0]];
    x1 = (float)((const _Float16*)x)[hd.coord[j0 + 1]];
  } else {
    x0 = ((const float*)x)[hd.coord[j0]];
    x1 = ((const float*)x)[hd.coord[j0 + 1]];
  }
  const float sq = x0 * x0 + x1 * x1;
  float ss[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) ss[k] = wave_sum(g == k ? sq : 0.f);
  const float nu = sqrtf(g == 0 ? ss[0] : g == 1 ? ss[1] : g == 2 ? ss[2] : ss[3]);
  ubuf[j0] = nu > 0.f ? x0 / nu : 0.f;
  ubuf[j0 + 1] = nu > 0.f ? x1 / nu : 0.f;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // y = Q^T u for this lane's two positions of its group (two rows per step into two sums
  // each, so that the reads of a step overlap; the group's dimension is even)
  float y0 = 0.f, y1 = 0.f, z0 = 0.f, z1 = 0.f;
  const float* q0 = rot + off + (j0 - st);
  for (int r = 0; r < n; r += 2) {
    const float2 u = *(const float2*)&ubuf[st + r];
    const float2 qa = *(const float2*)&q0[r * n], qb = *(const float2*)&q0[(r + 1) * n];
    y0 = fmaf(qa.x, u.x, y0);
    y1 = fmaf(qa.y, u.x, y1);
    z0 = fmaf(qb.x, u.y, z0);
    z1 = fmaf(qb.y, u.y, z1);
  }
  y0 += z0;
  y1 += z1;
  // compare-count against the group's boundaries
  const uint32_t c0 = count_below(y0, hd.boundary[g], nb), c1 = count_below(y1, hd.boundary[g], nb);
  if (PK == 1) {
    // bit l of m0 (m1) is the code of position 2l (2l + 1): word w interleaves bits
    // 16 w .. 16 w + 15 of both
    const uint64_t m0 = __builtin_amdgcn_ballot_w64(c0 != 0), m1 = __builtin_amdgcn_ballot_w64(c1 != 0);
    if (lane < 4)
      ((uint32_t*)code_rec)[lane] = spread_bits((uint32_t)(m0 >> (16 * lane)) & 0xFFFFu) |
                                    (spread_bits((uint32_t)(m1 >> (16 * lane)) & 0xFFFFu) << 1);
  } else if (PK == 2) {
    // byte k holds positions 4k .. 4k + 3: the 4-bit fields of lanes 2k and 2k + 1
    const uint32_t f = c0 | (c1 << 2), other = (uint32_t)__shfl_xor((int)f, 1);
    if (!(lane & 1)) code_rec[lane >> 1] = (uint8_t)(f | (other << 4));
  } else if (PK == 3) {
    // bytes 3k .. 3k + 2 hold positions 8k .. 8k + 7: the 6-bit fields of lanes 4k .. 4k + 3
    const int f = (int)(c0 | (c1 << 3)), q = lane & ~3;
    const uint32_t w = (uint32_t)__shfl(f, q) | ((uint32_t)__shfl(f, q + 1) << 6) | ((uint32_t)__shfl(f, q + 2) << 12) |
                       ((uint32_t)__shfl(f, q + 3) << 18);
    if ((lane & 3) < 3) code_rec[3 * (lane >> 2) + (lane & 3)] = (uint8_t)(w >> (8 * (lane & 3)));
  } else {
    if (hd.width[g] <= 4) {
      const int o = hd.byte_at[g] + ((j0 - st) >> 1);
      if (o < rec_bytes) code_rec[o] = (uint8_t)(c0 | (c1 << 4));
    } else {
      const int o = hd.byte_at[g] + (j0 - st);
      if (o < rec_bytes) code_rec[o] = (uint8_t)c0;
      if (o + 1 < rec_bytes) code_rec[o + 1] = (uint8_t)c1;
    }
    for (int i = hd.code_used + lane; i < rec_bytes; i += 64) code_rec[i] = 0;
  }
  float coef = 0.f;
  if (QJL) {
    const float e0 = y0 - hd.centroid[0][c0], e1 = y1 - hd.centroid[0][c1];
    // every lane's reads of u are complete (in-order LDS): e takes u's place
    ubuf[j0] = e0;
    ubuf[j0 + 1] = e1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float s0 = 0.f, s1 = 0.f;  // (M e)_i for i = lane and lane + 64
#pragma unroll 8
    for (int j = 0; j < 128; ++j) {
      const float e = ubuf[j];
      s0 = fmaf(proj[j * 128 + lane], e, s0);
      s1 = fmaf(proj[j * 128 + 64 + lane], e, s1);
    }
    const float ee = wave_sum(e0 * e0 + e1 * e1);
    const uint64_t b0 = __builtin_amdgcn_ballot_w64(s0 >= 0.f), b1 = __builtin_amdgcn_ballot_w64(s1 >= 0.f);
    if (lane < 4) ((uint32_t*)sign_rec)[lane] = (uint32_t)((lane < 2 ? b0 : b1) >> (32 * (lane & 1)));
    coef = 1.2533141373155003f / 128.f * sqrtf(ss[0]) * sqrtf(ee);  // sqrt(pi/2)/m |x| |e|
  }
  if (lane < 4) norm_rec[lane] = QJL && lane == 1 ? coef : lane < hd.n_groups ? sqrtf(ss[lane & 3]) : 0.f;
}

// ---------------------------------------------------------------------------------------
// Key encoding.  One workgroup per (512-token chunk, KV head, sequence) stages the head's
// encoder and rotations in LDS once; each wave encodes one token at a time: lane l holds
// group-order positions 2l and 2l + 1 (always in one group: groups start at even positions
// and have even sizes).
constexpr int kQuantTokens = 512;
template <bool XF16, bool QJL, int PK>
__global__ __launch_bounds__(256) void gtq_quantize_kernel(const GtqQuantArgs a) {
  const int CREC = PK ? 16 * PK : a.code_bytes;  // code bytes per key
  __shared__ __attribute__((aligned(16))) float rot[TQ_GTQ_ROTATION_FLOATS];
  __shared__ __attribute__((aligned(16))) float projl[QJL ? 128 * 128 : 1];
  __shared__ __attribute__((aligned(16))) float ubuf[4][128];
  __shared__ tq_gtq_head hd;
  const int tile = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  stage_head(&hd, (const tq_gtq_head*)a.heads + h);
  __syncthreads();
  int used = 0;
  for (int g = 0; g < hd.n_groups; ++g) used = hd.rot_offset[g] + hd.dim[g] * hd.dim[g];
  const float* grot = a.rotations + (size_t)h * TQ_GTQ_ROTATION_FLOATS;
  for (int i = tid; i < used; i += 256) rot[i] = grot[i];
  if (QJL)
    for (int i = tid; i < 128 * 128; i += 256) projl[i] = a.proj[(size_t)h * 128 * 128 + i];
  __syncthreads();

  const size_t stream = (size_t)b * a.n_kv_heads + h;
  for (int t = wv; t < kQuantTokens; t += 4) {
    const int i = tile * kQuantTokens + t;
    if (i >= a.n_new) break;
    const size_t rec = stream * a.capacity + a.pos0 + i;
    encode_key<XF16, QJL, PK>(hd, rot, (const uint8_t*)a.x + (stream * a.n_new + i) * 128 * (XF16 ? 2 : 4),
                              ubuf[wv], a.codes + rec * CREC, a.norms + rec * 4, lane, projl,
                              QJL ? a.signs + rec * 16 : nullptr, CREC);
    // the next token's writes to ubuf follow this token's reads in program order
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------------------
// Decode attention over Block-GTQ keys and fp16 values on the matrix unit (fp16 operands,
// fp32 accumulation, the page's tensor-core form).  One workgroup of NW waves per
// (sequence, KV head, section, slice of up to 8 query heads).  The section's 16-token tiles
// go to the waves in turn; each wave streams its tiles through its own ring of D LDS stages
// with direct global -> LDS copies (a stage: the 16 key records, their group norms, the 16
// fp16 value rows).
//
// Scores: the query is rotated per group in the prologue (q~ = Q_g^T q_g, scale and log2 e
// folded in) and laid out in k-blocks of 32 positions that each belong to one group (a
// group of n positions takes ceil(n/32) blocks; query positions past the group are zero,
// so the codes of the next group that share the block contribute nothing), divided by the
// group codebook's fp16 scale s and split into fp16 hi + lo columns.  The block's table
// holds, per code byte, the fp16 hi parts of s c for its two codes and then their lo
// parts, so a key operand is [hi pair, lo pair] of two bytes (four codes of one token)
// straight from two table reads, against a query operand that holds each position pair
// twice; two products cover a lane's 8 codes of the block with both key parts (scores
// keep fp32-level accuracy).  Each block's partial dot is multiplied by the token's group
// norm.  Tables sit at fixed LDS offsets per block and the norms group-major, so the
// unrolled block loop has no branch, mask or per-lane index beyond the code bytes.  The
// lazy softmax and the merge of waves are those of the codec kernel; the output product
// is a 16x16x16 one: weights as fp16 hi + lo rows straight from the lanes' score registers
// (k slots 4j .. 4j+3 = the lane's tokens), values of 4 tokens per lane read 8 bytes (4
// coordinates) at a time and paired by byte permutes, so tile ct holds coordinate
// 64 (ct / 4) + 4 col + ct % 4.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(u32x4 x, u32x4 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, x), __builtin_bit_cast(half8_t, y), c, 0,
                                                0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16_k16(u32x2 x, u32x2 y, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(half4_t, x), __builtin_bit_cast(half4_t, y), c, 0, 0,
                                               0);
}
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  return __builtin_bit_cast(uint32_t, half2_t{(_Float16)x, (_Float16)y});
}
__device__ __forceinline__ float f16_lo(float x) { return x - (float)(_Float16)x; }

constexpr float kRescaleG = 8.f;  // log2 headroom of the lazily updated softmax reference
constexpr int kMaxKb = 7;         // k-blocks of a head: sum over groups of ceil(n/32) <= 7

// QJL: two-stage keys (one MSE group plus sign bits of the projected residual): four more
// k-blocks whose key operands are +-1 (exact in fp16, from a table indexed by a sign byte)
// against the projected query S q = M Q^T q, times the coefficient in norm slot 1.
// PK: the first stage's width (1 to 3), its codes bit-packed in 16 PK bytes per key.
// PK = 1: the two levels c0 < c1 are written as mid + half (2 bit - 1), so
// <q~, c[code]> = mid sum_j q~_j + half sum_j q~_j (+-1)_j: four more +-1 products against
// half q~, plus mid sum_j q~_j added per head, replace the pair tables.  PK = 2: one table of
// 256 entries, a code byte's four codes as [hi pair, lo pair, hi pair, lo pair] (one 16-byte
// read per four codes).  PK = 3: one table of 64 entries over two codes, [hi pair, lo pair],
// read four times per lane's 24-bit word.
// WIDE (Block-GTQ records of more than 64 code bytes, with byte-container groups): the
// stage holds 2 KB of key records (two copies per stage); k-blocks of byte groups read the
// lane's 8 code bytes and decode each through its group's 256-entry table of [hi, lo] fp16
// parts, paired into operands by byte permutes.
template <int NW, int D, bool QF16, bool QJL, int PK = 0, bool WIDE = false>
__global__ __launch_bounds__(64 * NW) void gtq_attention_kernel(const GtqAttnArgs a) {
  static_assert((PK != 0) == QJL && PK >= 0 && PK <= 3, "packed codes are the first stage of two-stage keys");
  static_assert(!WIDE || PK == 0, "byte containers are Block-GTQ records");
  constexpr bool B1 = PK == 1;
  const int CREC = PK ? 16 * PK : WIDE ? a.code_bytes : 64;  // code bytes per key
  // a stage: key records 1 KB (2 KB when WIDE), norms 256 B (group-major), values 4 KB,
  // sign bytes 256 B
  constexpr int KAREA = WIDE ? 2048 : 1024;
  constexpr int NORM_AT = KAREA, VAL_AT = KAREA + 256, SIGN_AT = KAREA + 4352;
  constexpr int STAGE = QJL ? SIGN_AT + 256 : SIGN_AT;
  constexpr int NDMA = (QJL ? 7 : 6) + (WIDE ? 1 : 0);
  constexpr int WAVE_LDS = D * STAGE;
  static_assert(D >= 2 && D * NDMA <= 63, "ring depth within the memory counter");
  static_assert(NW == 4 || NW == 8, "the query rotation maps 64 NW threads onto 128 positions x 8 heads");
  // k-blocks: up to 7 for a Block-GTQ head; two-stage keys have one group of 128 (4 blocks)
  constexpr int KB = QJL ? 4 : kMaxKb;
  constexpr int PTAB_BYTES = PK == 0 ? KB * 256 * 8 : PK == 2 ? 256 * 16 : PK == 3 ? 64 * 8 : 0;
  constexpr int WTAB_BYTES = WIDE ? TQ_GTQ_MAX_GROUPS * 256 * 4 : 0;
  constexpr int TAB_BYTES = PTAB_BYTES + WTAB_BYTES + (QJL ? 256 * 16 : 0);  // pair tables, byte tables, +-1 table
  // the pair tables first, so that their addresses fit the LDS instructions' offset field
  __shared__ __attribute__((aligned(16))) uint8_t lds_all[TAB_BYTES + NW * WAVE_LDS];
  uint2(*const ptab)[256] = (uint2(*)[256])lds_all;
  uint8_t* const lds = lds_all + TAB_BYTES;
  uint8_t* const pmtab = lds_all + PTAB_BYTES + WTAB_BYTES;  // QJL: byte -> 8 fp16 +-1 (bit e: position e)
  // WIDE: per group, a byte code's level as fp16 hi | fp16 lo << 16 (zero past the codebook)
  uint32_t(*const wtab)[256] = (uint32_t(*)[256])(lds_all + PTAB_BYTES);
  // (ptab: per k-block and byte, the fp16 hi parts of s c for the byte's two codes, then
  // their lo parts; zero for the blocks past the head's last, which then add nothing.
  // PK = 2, 3: the one group's table, ptab4 or ptab6, at the same place)
  u32x4* const ptab4 = (u32x4*)lds_all;
  uint2* const ptab6 = (uint2*)lds_all;
  __shared__ __attribute__((aligned(16))) float qt[8][128];  // rotated, scaled query, group order
  __shared__ float qraw[8][128];  // the slice's query rows, original coordinates
  __shared__ tq_gtq_head hd;
  __shared__ float part_m[NW][8], part_l[NW][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int unit = blockIdx.x / a.n_slices, slice = blockIdx.x - unit * a.n_slices;
  const int split = unit % a.n_splits, kv = (unit / a.n_splits) % a.n_kv_heads;
  const int b = unit / (a.n_splits * a.n_kv_heads);
  const int h0 = kv * a.group_size + slice * a.heads_per_slice;
  const int hs = min(a.heads_per_slice, a.group_size - slice * a.heads_per_slice);
  const int T = a.seq_lens ? max(0, min(a.seq_lens[b] + a.len_bias, a.max_len)) : a.max_len;
  const int C = (T + a.n_splits - 1) / a.n_splits;
  const int lo = min(T, split * C), hi = min(T, lo + C);
  const int ntiles = lo < hi ? (hi - lo + 15) >> 4 : 0;
  const int n = ntiles > wv ? (ntiles - wv + NW - 1) / NW : 0;  // this wave's tiles

  const size_t row0 = ((size_t)b * a.n_kv_heads + kv) * a.capacity;
  const uint8_t* kc = a.codes + row0 * CREC;
  const uint8_t* kn = (const uint8_t*)(a.norms + row0 * 4);
  const uint8_t* vbp = (const uint8_t*)a.v + row0 * 256;
  const uint8_t* sgb = QJL ? a.signs + row0 * 16 : nullptr;
  const int cap = a.capacity;
  uint8_t* wlds = lds + wv * WAVE_LDS;
  const uint32_t wlds_a = lds_addr(wlds);

  auto tok0_of = [&](int s) { return lo + 16 * (wv + NW * s); };
  // stage s: 16 key records (lane: token tok0 + l/4, 16 bytes), the 64 norms group-major
  // (lane: group l/16 of token tok0 + l%16), 16 value rows (4 copies; lane: token
  // tok0 + 4k + l/16); tokens past the capacity are replaced by the tile's first token
  // (their weights are 0)
  auto issue = [&](int s) {
    const int t0 = tok0_of(s);
    const uint32_t dst = wlds_a + (s % D) * STAGE;
    int t = t0 + (lane >> 2);
    if (B1) {  // 16 tokens' code bytes (lane: token tok0 + l/4, 4 bytes)
      lds_dma<4, true>(dst, kc, t < cap ? (uint32_t)(t * 16 + 4 * (lane & 3)) : (uint32_t)(t0 * 16));
    } else if (PK) {
      // the 16 tokens' 16 PK-byte records are one span: lane l copies its bytes 16 l .. + 15
      // (token tok0 + l / PK); lanes past the span repeat the first lanes into the stage's
      // unused key bytes
      const int l = lane % (16 * PK);
      t = t0 + l / PK;
      lds_dma<16, true>(dst, kc, t < cap ? (uint32_t)(t * CREC + 16 * (l % PK)) : (uint32_t)(t0 * CREC));
    } else if (WIDE) {
      // the 16 records (CREC bytes each, a multiple of 16) are one span: copy d moves its
      // bytes 1024 d + 16 l .. + 15; lanes past the span read the tile's first record
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int o = 1024 * d + 16 * lane, tk = o / CREC;
        t = t0 + tk;
        lds_dma<16, true>(dst + 1024 * d, kc,
                          tk < 16 && t < cap ? (uint32_t)(t * CREC + (o - tk * CREC)) : (uint32_t)(t0 * CREC));
      }
    } else {
      lds_dma<16, true>(dst, kc, t < cap ? (uint32_t)(t * 64 + 16 * (lane & 3)) : (uint32_t)(t0 * 64));
    }
    t = t0 + (lane & 15);
    lds_dma<4, true>(dst + NORM_AT, kn, t < cap ? (uint32_t)(t * 16 + 4 * (lane >> 4)) : (uint32_t)(t0 * 16));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      t = t0 + 4 * k + (lane >> 4);
      lds_dma<16, true>(dst + VAL_AT + 1024 * k, vbp,
                        t < cap ? (uint32_t)t * 256u + 16u * (lane & 15) : (uint32_t)t0 * 256u);
    }
    if (QJL) {  // 16 tokens' sign bytes (lane: token tok0 + l/4, 4 bytes)
      t = t0 + (lane >> 2);
      lds_dma<4, true>(dst + SIGN_AT, sgb, t < cap ? (uint32_t)(t * 16 + 4 * (lane & 3)) : (uint32_t)(t0 * 16));
    }
  };

  // prologue: the head's encoder and the slice's query rows (one round trip), then the
  // k-block plan, the pair tables and the rotated query
  stage_head_part<WIDE ? 256 : 16>(&hd, (const tq_gtq_head*)a.heads + kv);
  for (int i = tid; i < 8 * 128; i += 64 * NW) {
    const int hh = i >> 7, c = i & 127;
    const size_t qi = ((size_t)b * a.n_q_heads + h0 + hh) * 128 + c;
    qraw[hh][c] = hh >= hs ? 0.f : QF16 ? (float)((const _Float16*)a.q)[qi] : ((const float*)a.q)[qi];
  }
  __syncthreads();
  // Fused append: if this workgroup's section holds the row's new slot, wave 0 writes that
  // token's key record and value row (reading the rotations from global memory, with its
  // own ring space as scratch) while the other waves build the tables; the barrier below
  // orders its stores before any copy of the cache.  Other sections do not read the slot.
  if (a.append && wv == 0) {
    const int p = a.seq_lens ? a.seq_lens[b] : a.max_len - 1;  // the new slot: rows end at it
    if (p >= 0 && p < a.max_len && p >= lo && p < hi) {
      const size_t st = (size_t)b * a.n_kv_heads + kv, rec = st * a.capacity + p;
      const float* grot = a.rotations + (size_t)kv * TQ_GTQ_ROTATION_FLOATS;
      _Float16* vd = (_Float16*)a.w_v + rec * 128;
      // two-stage keys: also the sign bits (M^T read from global memory)
      const float* pj = QJL ? a.proj + (size_t)kv * 128 * 128 : nullptr;
      uint8_t* srec = QJL ? a.w_signs + rec * 16 : nullptr;
      if (a.x_f16) {
        encode_key<true, QJL, PK>(hd, grot, (const _Float16*)a.k_new + st * 128, (float*)wlds,
                                  a.w_codes + rec * CREC, a.w_norms + rec * 4, lane, pj, srec, CREC);
        ((uint32_t*)vd)[lane] = ((const uint32_t*)a.v_new)[st * 64 + lane];
      } else {
        encode_key<false, QJL, PK>(hd, grot, (const float*)a.k_new + st * 128, (float*)wlds,
                                   a.w_codes + rec * CREC, a.w_norms + rec * 4, lane, pj, srec, CREC);
        const float2 x = ((const float2*)a.v_new)[st * 64 + lane];
        ((uint32_t*)vd)[lane] = pack_f16(x.x, x.y);
      }
    }
  }
  // The k-block plan, uniform and in registers: group g takes blocks cum[g] .. cum[g+1]-1
  // (ceil(dim_g / 32) of them), so block kb belongs to the group whose range holds it.
  int cum[TQ_GTQ_MAX_GROUPS + 1];
  {
    const int ng = min(__builtin_amdgcn_readfirstlane(hd.n_groups), TQ_GTQ_MAX_GROUPS);
    cum[0] = 0;
#pragma unroll
    for (int g = 0; g < TQ_GTQ_MAX_GROUPS; ++g)
      cum[g + 1] = cum[g] + (g < ng ? (__builtin_amdgcn_readfirstlane(hd.dim[g]) + 31) / 32 : 0);
  }
  const int nkb = min(cum[TQ_GTQ_MAX_GROUPS], KB);
  auto group_of_block = [&](int kb) { return (kb >= cum[1]) + (kb >= cum[2]) + (kb >= cum[3]); };
  for (int i = tid; i < (PK ? 0 : KB * 256); i += 64 * NW) {
    const int kb = i >> 8, by = i & 255, g = kb < nkb ? group_of_block(kb) : 0;
    // codes past the codebook decode to 0 (and byte groups do not use these tables)
    const int nc = kb < nkb && hd.width[g] <= 4 ? 1 << max(hd.width[g], 1) : 0;
    const float sc = hd.f16_scale[g];
    const float c0 = (by & 15) < nc ? sc * hd.centroid[g][by & 15] : 0.f;
    const float c1 = (by >> 4) < nc ? sc * hd.centroid[g][by >> 4] : 0.f;
    ptab[kb][by] = make_uint2(pack_f16(c0, c1), pack_f16(f16_lo(c0), f16_lo(c1)));
  }
  if (WIDE) {
    for (int i = tid; i < TQ_GTQ_MAX_GROUPS * 256; i += 64 * NW) {
      const int g = i >> 8, c = i & 255;
      const int nc = g < hd.n_groups && hd.width[g] > 4 ? 1 << min(hd.width[g], 8) : 0;
      const float v = c < nc ? hd.f16_scale[g] * hd.centroid[g][c] : 0.f;
      wtab[g][c] = pack_f16(v, f16_lo(v));
    }
  }
  if (PK == 2 || PK == 3) {  // the one group's levels (codes past its codebook decode to 0)
    const int nc = 1 << min(max(hd.width[0], 1), PK);
    const float sc = hd.f16_scale[0];
    auto lev = [&](int c) { return c < nc ? sc * hd.centroid[0][c] : 0.f; };
    for (int i = tid; i < (PK == 2 ? 256 : 64); i += 64 * NW) {
      if (PK == 2) {
        const float c0 = lev(i & 3), c1 = lev((i >> 2) & 3), c2 = lev((i >> 4) & 3), c3 = lev(i >> 6);
        ptab4[i] = u32x4{pack_f16(c0, c1), pack_f16(f16_lo(c0), f16_lo(c1)), pack_f16(c2, c3),
                         pack_f16(f16_lo(c2), f16_lo(c3))};
      } else {
        const float c0 = lev(i & 7), c1 = lev(i >> 3);
        ptab6[i] = make_uint2(pack_f16(c0, c1), pack_f16(f16_lo(c0), f16_lo(c1)));
      }
    }
  }
  {
    // q~_g = Q_g^T q_g: thread (j, k) takes group-order position j of heads k, k + NW/2, ..,
    // which share the rotation column Q_g[:, j]
    const float* grot = a.rotations + (size_t)kv * TQ_GTQ_ROTATION_FLOATS;
    constexpr int HK = 16 / NW;  // heads per thread
    const int j = tid & 127, k0 = tid >> 7;
    const int g = group_of(hd, j), s0 = hd.start[g], nd = hd.dim[g];
    const float* rr = grot + hd.rot_offset[g] + (j - s0);
    float acc[HK];
#pragma unroll
    for (int e = 0; e < HK; ++e) acc[e] = 0.f;
#pragma unroll 16
    for (int r = 0; r < nd; ++r) {
      const float w = rr[r * nd];
      const int c = hd.coord[s0 + r];
#pragma unroll
      for (int e = 0; e < HK; ++e) acc[e] = fmaf(w, qraw[k0 + (NW / 2) * e][c], acc[e]);
    }
    const float f = a.scale_log2 / hd.f16_scale[g];
#pragma unroll
    for (int e = 0; e < HK; ++e) qt[k0 + (NW / 2) * e][j] = acc[e] * f;
  }
  if (QJL) {  // the +-1 table: entry by, fp16 pair k = (bit 2k, bit 2k + 1) of by, 1 -> +1
    for (int i = tid; i < 256 * 4; i += 64 * NW) {
      const int by = i >> 2, k = i & 3;
      ((uint32_t*)pmtab)[i] = pack_f16((by >> (2 * k)) & 1 ? 1.f : -1.f, (by >> (2 * k + 1)) & 1 ? 1.f : -1.f);
    }
  }
  __syncthreads();
  const int col = lane & 15;
  const int jr = lane >> 4;
  // QJL: the projected query w = M q~ (q~ = Q^T q, already scaled in qt by scale_log2 / s,
  // so w is scaled back by s) into qraw, then its operands: block m's positions
  // 32 m + 8 jr .. + 7, fp16 hi (columns 0-7) and lo (8-15) parts
  u32x4 qq[QJL ? 4 : 1];
  if (QJL) {
    const int i = tid & 127, k0 = tid >> 7;
    constexpr int HK = 16 / NW;
    const float* pj = a.proj + (size_t)kv * 128 * 128;
    float acc[HK];
#pragma unroll
    for (int e = 0; e < HK; ++e) acc[e] = 0.f;
#pragma unroll 16
    for (int jj = 0; jj < 128; ++jj) {
      const float w = pj[jj * 128 + i];
#pragma unroll
      for (int e = 0; e < HK; ++e) acc[e] = fmaf(w, qt[k0 + (NW / 2) * e][jj], acc[e]);
    }
    const float s0 = hd.f16_scale[0];
#pragma unroll
    for (int e = 0; e < HK; ++e) qraw[k0 + (NW / 2) * e][i] = acc[e] * s0;
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = qraw[col & 7][32 * m + 8 * jr + 2 * e], v1 = qraw[col & 7][32 * m + 8 * jr + 2 * e + 1];
        x[e] = col >= 8 ? pack_f16(f16_lo(v0), f16_lo(v1)) : pack_f16(v0, v1);
      }
      qq[m] = u32x4{x[0], x[1], x[2], x[3]};
    }
  }
  // B1: half s q~ as +-1 operands (block m's positions 32 m + 8 jr .. + 7, fp16 hi in columns
  // 0-7, lo in 8-15) and mid s sum_j q~_j for the hi columns (qt holds q~ / s)
  u32x4 qm[B1 ? 4 : 1];
  float moff = 0.f;
  if (B1) {
    const float s0 = hd.f16_scale[0], c0 = hd.centroid[0][0], c1 = hd.centroid[0][1];
    const float hf = 0.5f * (c1 - c0) * s0, md = 0.5f * (c0 + c1) * s0;
    float part = 0.f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = qt[col & 7][32 * m + 8 * jr + 2 * e], v1 = qt[col & 7][32 * m + 8 * jr + 2 * e + 1];
        part += v0 + v1;
        x[e] = col >= 8 ? pack_f16(f16_lo(hf * v0), f16_lo(hf * v1)) : pack_f16(hf * v0, hf * v1);
      }
      qm[m] = u32x4{x[0], x[1], x[2], x[3]};
    }
    part = sum_rows(part);
    moff = col < 8 ? md * part : 0.f;
  }
  // query operands: block kb's positions 8 jr .. + 3 (qa) and + 4 .. + 7 (qb), each pair
  // twice, matching key operands [hi pair, lo pair, hi pair, lo pair]; and per block its
  // group (uniform) and the byte of the lane's first code (reads past a record's 64 bytes
  // stay inside the stage and meet zero query)
  u32x4 qa[KB], qb[KB];
  int kgrp[KB];
  uint32_t kbyte[KB];
  bool kwide[KB];  // WIDE: the block's group has byte containers (uniform)
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const int g = kb < nkb ? group_of_block(kb) : 0, m = kb < nkb ? kb - cum[g] : 0;
    const int dg = hd.dim[g], sg = hd.start[g];
    kgrp[kb] = g;
    kwide[kb] = WIDE && kb < nkb && __builtin_amdgcn_readfirstlane(hd.width[g]) > 4;
    // nibble groups: byte (position) / 2; byte groups: one byte per position from byte_at
    kbyte[kb] = kwide[kb] ? (uint32_t)(hd.byte_at[g] + 32 * m + 8 * jr) : (uint32_t)((sg + 32 * m + 8 * jr) >> 1);
    qa[kb] = qb[kb] = u32x4{0u, 0u, 0u, 0u};
    if (!B1 && kb < nkb) {
      const int hh = col & 7;
      uint32_t x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int p = 32 * m + 8 * jr + 2 * e;
        const float v0 = p < dg ? qt[hh][sg + p] : 0.f;
        const float v1 = p + 1 < dg ? qt[hh][sg + p + 1] : 0.f;
        x[e] = col >= 8 ? pack_f16(f16_lo(v0), f16_lo(v1)) : pack_f16(v0, v1);
      }
      qa[kb] = u32x4{x[0], x[0], x[1], x[1]};
      qb[kb] = u32x4{x[2], x[2], x[3], x[3]};
    }
  }
  if (!B1) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) asm volatile("" ::"v"(qa[kb]), "v"(qb[kb]));
  }
  vm_wait<0>();
  for (int s = 0; s < D; ++s)
    if (s < n) issue(s);

  f32x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, thr = -INFINITY, lsum = 0.f;

  for (int s = 0; s < n; ++s) {
    const int younger = min(D - 1, n - 1 - s);
    if (younger >= 3) vm_wait<3 * NDMA>();
    else if (younger == 2) vm_wait<2 * NDMA>();
    else if (younger == 1) vm_wait<NDMA>();
    else vm_wait<0>();
    const int t0 = tok0_of(s);
    const int nv = min(16, hi - t0);
    const uint8_t* sb = wlds + (s % D) * STAGE;

    // ---- scores: the key operand row is token col; lane's k slots are codes 8 jr .. + 7
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (B1) {  // code bytes as +-1 operands against half q~, then + mid sum q~, times the norm
      f32x4 cm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t by = lds_read<uint8_t>(sb + 16 * col + 4 * m + jr);
        cm = mfma_f16(lds_read<u32x4>(pmtab + 16 * by), qm[m], cm);
      }
      const float4 nr = lds_read<float4>(sb + NORM_AT + 16 * jr);
      sc[0] = nr.x * (cm[0] + moff);
      sc[1] = nr.y * (cm[1] + moff);
      sc[2] = nr.z * (cm[2] + moff);
      sc[3] = nr.w * (cm[3] + moff);
    } else {
      const uint8_t* rec = sb + CREC * col;
      // every block is computed (those past the head's last have zero tables and query), so
      // the unrolled loop is one basic block the compiler can interleave
      uint32_t cb[KB], cb2[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {  // every code word first
        cb2[kb] = 0u;
        if (WIDE && kwide[kb]) {  // the lane's 8 code bytes from three aligned words
          const uint32_t bo = kbyte[kb];
          const uint32_t w0 = lds_read<uint32_t>(rec + (bo & ~3u)), w1 = lds_read<uint32_t>(rec + (bo & ~3u) + 4),
                         w2 = lds_read<uint32_t>(rec + (bo & ~3u) + 8);
          cb[kb] = __builtin_amdgcn_alignbyte(w1, w0, bo & 3u);
          cb2[kb] = __builtin_amdgcn_alignbyte(w2, w1, bo & 3u);
        } else if (PK == 2) {  // positions 32 kb + 8 jr .. + 7: two bytes
          cb[kb] = lds_read<uint16_t>(rec + 8 * kb + 2 * jr);
        } else {
          // the lane's code bytes (4 nibble bytes, or the 3 bytes of a 24-bit word at
          // 12 kb + 3 jr) from two aligned words (the byte offset is any multiple of 1)
          const uint32_t bo = PK == 3 ? (uint32_t)(12 * kb + 3 * jr) : kbyte[kb];
          const uint32_t w0 = lds_read<uint32_t>(rec + (bo & ~3u)), w1 = lds_read<uint32_t>(rec + (bo & ~3u) + 4);
          cb[kb] = __builtin_amdgcn_alignbyte(w1, w0, bo & 3u);
        }
      }
      // key operands straight from the table reads: [hi pair, lo pair] of two codes each
      u32x4 ka[KB], kb2[KB];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        if (PK == 2) {
          ka[kb] = ptab4[cb[kb] & 255u];
          kb2[kb] = ptab4[(cb[kb] >> 8) & 255u];
        } else if (PK == 3) {
          const uint2 e0 = ptab6[cb[kb] & 63u], e1 = ptab6[(cb[kb] >> 6) & 63u];
          const uint2 e2 = ptab6[(cb[kb] >> 12) & 63u], e3 = ptab6[(cb[kb] >> 18) & 63u];
          ka[kb] = u32x4{e0.x, e0.y, e1.x, e1.y};
          kb2[kb] = u32x4{e2.x, e2.y, e3.x, e3.y};
        } else if (WIDE && kwide[kb]) {
          // one code per byte: [hi, lo] words paired by permutes into [hi pair, lo pair]
          const uint32_t* wt = wtab[kgrp[kb]];
          uint32_t e[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[i] = wt[(cb[kb] >> (8 * i)) & 255u];
            e[4 + i] = wt[(cb2[kb] >> (8 * i)) & 255u];
          }
          ka[kb] = u32x4{__builtin_amdgcn_perm(e[1], e[0], 0x05040100u), __builtin_amdgcn_perm(e[1], e[0], 0x07060302u),
                         __builtin_amdgcn_perm(e[3], e[2], 0x05040100u), __builtin_amdgcn_perm(e[3], e[2], 0x07060302u)};
          kb2[kb] = u32x4{__builtin_amdgcn_perm(e[5], e[4], 0x05040100u), __builtin_amdgcn_perm(e[5], e[4], 0x07060302u),
                          __builtin_amdgcn_perm(e[7], e[6], 0x05040100u), __builtin_amdgcn_perm(e[7], e[6], 0x07060302u)};
        } else {
          const uint2 e0 = ptab[kb][cb[kb] & 255u], e1 = ptab[kb][(cb[kb] >> 8) & 255u];
          const uint2 e2 = ptab[kb][(cb[kb] >> 16) & 255u], e3 = ptab[kb][cb[kb] >> 24];
          ka[kb] = u32x4{e0.x, e0.y, e1.x, e1.y};
          kb2[kb] = u32x4{e2.x, e2.y, e3.x, e3.y};
        }
      }
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        // (c_hi + c_lo) (q_hi + q_lo): both key parts against both query columns
        f32x4 cur = mfma_f16(ka[kb], qa[kb], f32x4{0.f, 0.f, 0.f, 0.f});
        cur = mfma_f16(kb2[kb], qb[kb], cur);
        // times the group norms of the lane's tokens 4 jr .. + 3
        const float4 nr = lds_read<float4>(sb + NORM_AT + 64 * kgrp[kb] + 16 * jr);
        sc[0] = fmaf(nr.x, cur[0], sc[0]);
        sc[1] = fmaf(nr.y, cur[1], sc[1]);
        sc[2] = fmaf(nr.z, cur[2], sc[2]);
        sc[3] = fmaf(nr.w, cur[3], sc[3]);
      }
    }
    if (QJL) {  // the residual's estimate: sign operands against S q, times slot 1
      f32x4 cq = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t by = lds_read<uint8_t>(sb + SIGN_AT + 16 * col + 4 * m + jr);
        cq = mfma_f16(lds_read<u32x4>(pmtab + 16 * by), qq[m], cq);
      }
      const float4 nr = lds_read<float4>(sb + NORM_AT + 64 + 16 * jr);
      sc[0] = fmaf(nr.x, cq[0], sc[0]);
      sc[1] = fmaf(nr.y, cq[1], sc[1]);
      sc[2] = fmaf(nr.z, cq[2], sc[2]);
      sc[3] = fmaf(nr.w, cq[3], sc[3]);
    }
    float x[4];
    float bm = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = sc[e] + dpp<0x128>(sc[e]);  // hi + lo query parts
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
      thr = mnew + kRescaleG;
    }
    u32x2 pf;
    {
      float pw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[e] = __builtin_amdgcn_exp2f(x[e] - mref);
        lsum += pw[e];
        if (col >= 8) pw[e] = f16_lo(pw[e]);
      }
      pf = u32x2{pack_f16(pw[0], pw[1]), pack_f16(pw[2], pw[3])};
    }
    // ---- output: values of tokens 4 jr .. + 3; tile ct holds coordinate
    // 64 (ct / 4) + 4 col + ct % 4, so one 8-byte read per token serves four tiles
    u32x2 vw[8];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      uint2 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = lds_read<uint2>(sb + VAL_AT + 256 * (4 * jr + e) + 128 * u + 8 * col);
      // tile 4u + j: [v(t0, j), v(t1, j)], [v(t2, j), v(t3, j)]
      vw[4 * u + 0] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, 0x05040100u), __builtin_amdgcn_perm(r[3].x, r[2].x, 0x05040100u)};
      vw[4 * u + 1] = u32x2{__builtin_amdgcn_perm(r[1].x, r[0].x, 0x07060302u), __builtin_amdgcn_perm(r[3].x, r[2].x, 0x07060302u)};
      vw[4 * u + 2] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, 0x05040100u), __builtin_amdgcn_perm(r[3].y, r[2].y, 0x05040100u)};
      vw[4 * u + 3] = u32x2{__builtin_amdgcn_perm(r[1].y, r[0].y, 0x07060302u), __builtin_amdgcn_perm(r[3].y, r[2].y, 0x07060302u)};
    }
    if (nv < 16) {  // a partial tile: tokens past the row carry zeros (their weights are 0)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const int t = 4 * jr;
        vw[ct].x &= (t < nv ? 0xFFFFu : 0u) | (t + 1 < nv ? 0xFFFF0000u : 0u);
        vw[ct].y &= (t + 2 < nv ? 0xFFFFu : 0u) | (t + 3 < nv ? 0xFFFF0000u : 0u);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[ct] = mfma_f16_k16(pf, vw[ct], acc[ct]);
    if (s + D < n) {
      lds_wait();
      issue(s + D);
    }
  }

  // ---- merge the waves
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
    const float o = L > 0.f ? O / L : 0.f;
    const float lse = L > 0.f ? (M + __log2f(L)) * kLn2g : -INFINITY;
    if (a.n_splits == 1) {
      const size_t row = (size_t)b * a.n_q_heads + h0 + h;
      a.out[row * 128 + c] = o;
      if (c == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      const size_t row = ((size_t)split * a.batch + b) * a.n_q_heads + h0 + h;
      a.part_o[row * 128 + c] = o;
      if (c == 0) a.part_lse[row] = lse;
    }
  }
}

}  // namespace

hipError_t launch_gtq_quantize(const GtqQuantArgs& a, bool x_f16, int batch, hipStream_t stream) {
  const dim3 grid((a.n_new + kQuantTokens - 1) / kQuantTokens, a.n_kv_heads, batch), block(256);
  if ((a.code_bits != 0) != (a.signs != nullptr) || a.code_bits < 0 || a.code_bits > 3) return hipErrorInvalidValue;
  if (a.code_bits == 0 && (a.code_bytes < 64 || a.code_bytes > 128 || a.code_bytes % 16)) return hipErrorInvalidValue;
#define TQ_GQ(PK)                                                                                            \
  if (a.code_bits == PK) {                                                                                   \
    if (x_f16) hipLaunchKernelGGL((gtq_quantize_kernel<true, PK != 0, PK>), grid, block, 0, stream, a);      \
    else hipLaunchKernelGGL((gtq_quantize_kernel<false, PK != 0, PK>), grid, block, 0, stream, a);           \
  }
  TQ_GQ(0) TQ_GQ(1) TQ_GQ(2) TQ_GQ(3)
#undef TQ_GQ
  return hipGetLastError();
}

hipError_t launch_gtq_attention(const GtqAttnArgs& a, bool q_f16, hipStream_t stream) {
  constexpr int NW = 8, D = 2;
  const dim3 grid(a.batch * a.n_kv_heads * a.n_splits * a.n_slices), block(64 * NW);
  if (a.heads_per_slice > 8) return hipErrorInvalidValue;
  if ((a.code_bits != 0) != (a.signs != nullptr) || a.code_bits < 0 || a.code_bits > 3) return hipErrorInvalidValue;
  const bool wide = a.code_bits == 0 && a.code_bytes > 64;
  if (a.code_bits == 0 && (a.code_bytes < 64 || a.code_bytes > 128 || a.code_bytes % 16)) return hipErrorInvalidValue;
#define TQ_GA(PK, W)                                                                                                 \
  if (a.code_bits == PK && wide == W) {                                                                              \
    if (q_f16) hipLaunchKernelGGL((gtq_attention_kernel<NW, D, true, PK != 0, PK, W>), grid, block, 0, stream, a);   \
    else hipLaunchKernelGGL((gtq_attention_kernel<NW, D, false, PK != 0, PK, W>), grid, block, 0, stream, a);        \
  }
  TQ_GA(0, false) TQ_GA(0, true) TQ_GA(1, false) TQ_GA(2, false) TQ_GA(3, false)
#undef TQ_GA
  return hipGetLastError();
}

}  // namespace tq

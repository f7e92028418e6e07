// Host side of Block-GTQ keys ("RoPE-Aware Bit Allocation for KV-Cache Quantization"): the
// greedy integer bit allocation and the per-head encoder (groups of equal width, their
// uniformly random rotations and Lloyd-Max codebooks).
#include <cmath>
#include <cstring>
#include <vector>

#include "tq.h"

namespace tq {
// 5 .. 8-bit Lloyd-Max codebook (tq_codebook.cpp)
bool wide_codebook(int bits, int dim, float* centroid, float* boundary, float* scale);
}

extern "C" tq_status tq_gtq_block_energies(const float* q_cal, const float* k_cal, int32_t n_tokens,
                                           int32_t n_q_heads, int32_t n_kv_heads, float* energies) {
  if (q_cal == nullptr || k_cal == nullptr || energies == nullptr) return TQ_EINVAL;
  if (n_tokens <= 0 || n_q_heads <= 0 || n_kv_heads <= 0 || n_q_heads % n_kv_heads != 0) return TQ_EINVAL;
  const int g = n_q_heads / n_kv_heads;
  for (int h = 0; h < n_kv_heads; ++h) {
    for (int i = 0; i < TQ_GTQ_BLOCKS; ++i) {
      double sq = 0.0, sk = 0.0;
      for (int t = 0; t < n_tokens; ++t) {
        for (int r = 0; r < g; ++r) {
          const float* q = q_cal + ((size_t)t * n_q_heads + h * g + r) * 128 + 2 * i;
          sq += (double)q[0] * q[0] + (double)q[1] * q[1];
        }
        const float* k = k_cal + ((size_t)t * n_kv_heads + h) * 128 + 2 * i;
        sk += (double)k[0] * k[0] + (double)k[1] * k[1];
      }
      energies[h * TQ_GTQ_BLOCKS + i] = (float)(0.5 * (sq / ((double)n_tokens * g) + sk / n_tokens));
    }
  }
  return TQ_OK;
}

extern "C" tq_status tq_gtq_allocate(const float* energies, int32_t n_blocks, int32_t budget, int32_t b_min,
                                     int32_t b_max, int32_t* bits) {
  if (energies == nullptr || bits == nullptr || n_blocks <= 0) return TQ_EINVAL;
  if (b_min < 0 || b_max < b_min || b_max > 30) return TQ_EINVAL;
  if ((int64_t)budget < (int64_t)n_blocks * b_min || (int64_t)budget > (int64_t)n_blocks * b_max) return TQ_EINVAL;
  for (int i = 0; i < n_blocks; ++i)
    if (!(energies[i] >= 0.f) || !std::isfinite(energies[i])) return TQ_EINVAL;
  for (int i = 0; i < n_blocks; ++i) bits[i] = b_min;
  // each extra bit to the block with the largest gain (3/4) s 4^-b; 4^-b is a power of two,
  // so the gain is (0.75 s) rounded once, scaled exactly
  for (int64_t r = (int64_t)budget - (int64_t)n_blocks * b_min; r > 0; --r) {
    int best = -1;
    double gain = -1.0;
    for (int i = 0; i < n_blocks; ++i) {
      if (bits[i] >= b_max) continue;
      const double g = std::ldexp(0.75 * (double)energies[i], -2 * bits[i]);
      if (g > gain) {
        gain = g;
        best = i;
      }
    }
    bits[best] += 1;
  }
  return TQ_OK;
}

extern "C" tq_status tq_gtq_prepare(const int32_t* block_bits, const float* gauss, tq_gtq_head* head,
                                    float* rotation) {
  if (block_bits == nullptr || gauss == nullptr || head == nullptr || rotation == nullptr) return TQ_EINVAL;
  int present = 0;
  for (int i = 0; i < TQ_GTQ_BLOCKS; ++i) {
    if (block_bits[i] < 1 || block_bits[i] > TQ_GTQ_MAX_WIDTH) return TQ_EINVAL;
    present |= 1 << block_bits[i];
  }
  if (__builtin_popcount(present) > TQ_GTQ_MAX_GROUPS) return TQ_EUNSUPPORTED;
  std::memset(head, 0, sizeof(*head));
  std::memset(rotation, 0, sizeof(float) * TQ_GTQ_ROTATION_FLOATS);
  int pos = 0, off = 0, g = 0;
  for (int w = 1; w <= TQ_GTQ_MAX_WIDTH; ++w) {
    std::vector<int> coords;
    for (int i = 0; i < TQ_GTQ_BLOCKS; ++i)
      if (block_bits[i] == w) {
        coords.push_back(2 * i);
        coords.push_back(2 * i + 1);
      }
    if (coords.empty()) continue;
    const int n = (int)coords.size();
    head->width[g] = w;
    head->start[g] = pos;
    head->dim[g] = n;
    head->rot_offset[g] = off;
    for (int j = 0; j < n; ++j) head->coord[pos + j] = coords[j];
    // columns of the leading n x n part, orthonormalised in order (modified Gram-Schmidt):
    // the Q of the QR factorisation whose R has a positive diagonal
    std::vector<double> q((size_t)n * n);
    const float* a = gauss + (size_t)(w - 1) * 128 * 128;
    for (int c = 0; c < n; ++c) {
      std::vector<double> v(n);
      for (int r = 0; r < n; ++r) v[r] = a[r * 128 + c];
      for (int p = 0; p < c; ++p) {
        double d = 0.0;
        for (int r = 0; r < n; ++r) d += q[(size_t)r * n + p] * v[r];
        for (int r = 0; r < n; ++r) v[r] -= d * q[(size_t)r * n + p];
      }
      double nrm = 0.0;
      for (int r = 0; r < n; ++r) nrm += v[r] * v[r];
      nrm = std::sqrt(nrm);
      if (!(nrm > 0.0)) return TQ_EINVAL;
      for (int r = 0; r < n; ++r) q[(size_t)r * n + c] = v[r] / nrm;
    }
    for (int i = 0; i < n * n; ++i) rotation[off + i] = (float)q[i];
    if (w <= 4) {
      tq_codebook cb;
      const tq_status st = tq_make_codebook(w, n, &cb);
      if (st != TQ_OK) return st;
      for (int k = 0; k < 16; ++k) head->centroid[g][k] = cb.centroid[k];
      for (int k = 0; k < 15; ++k) head->boundary[g][k] = cb.boundary[k];
      head->f16_scale[g] = cb.f16_scale;
    } else if (!tq::wide_codebook(w, n, head->centroid[g], head->boundary[g], &head->f16_scale[g])) {
      return TQ_EUNSUPPORTED;
    }
    pos += n;
    off += n * n;
    ++g;
  }
  head->n_groups = g;
  for (int k = g; k < TQ_GTQ_MAX_GROUPS; ++k) head->start[k] = 128;
  // record layout: the nibble groups' P positions (two per byte), then a byte per position
  // of the wider groups
  int nib = 0;
  for (int k = 0; k < g; ++k)
    if (head->width[k] <= 4) nib += head->dim[k];
  for (int k = 0; k < g; ++k) head->byte_at[k] = head->width[k] <= 4 ? head->start[k] / 2 : nib / 2 + head->start[k] - nib;
  for (int k = g; k < TQ_GTQ_MAX_GROUPS; ++k) head->byte_at[k] = nib / 2 + 128 - nib;
  head->code_used = nib / 2 + 128 - nib;
  head->code_bytes = nib == 128 ? 64 : (head->code_used + 15) / 16 * 16;
  return TQ_OK;
}

extern "C" tq_status tq_gtq_qjl_projection(const tq_gtq_head* head, const float* rotation, const float* S,
                                           float* proj) {
  if (head == nullptr || rotation == nullptr || S == nullptr || proj == nullptr) return TQ_EINVAL;
  // the two-stage keys' first stage is one group of all 128 coordinates in order
  if (head->n_groups != 1 || head->dim[0] != 128 || head->rot_offset[0] != 0) return TQ_EINVAL;
  for (int j = 0; j < 128; ++j)
    if (head->coord[j] != j) return TQ_EINVAL;
  // M = S Q in double; stored transposed: proj[j][i] = M[i][j]
  for (int i = 0; i < 128; ++i)
    for (int j = 0; j < 128; ++j) {
      double acc = 0.0;
      for (int c = 0; c < 128; ++c) acc += (double)S[i * 128 + c] * (double)rotation[c * 128 + j];
      proj[j * 128 + i] = (float)acc;
    }
  return TQ_OK;
}

// C ABI of the packed-KV decode attention library: argument checks on the host, then one
// launch per call on the caller's stream.  No allocation; the only state is per-device (the
// compute-unit count, and the static partial buffer's address).
#include <cmath>
#include <cstdint>
#include <cstring>

#include "tq.h"
#include "tq_internal.h"

namespace {

bool valid_codebook(const tq_codebook& cb, int bits, int group) {
  return cb.bits == bits && cb.dim == group && cb.f16_scale >= 1.f && cb.f16_scale < 2.f;
}

tq_status check_rotation(const tq_rotation* rot) {
  if (rot == nullptr || rot->signs == nullptr) return TQ_EINVAL;
  if (rot->n_kv_heads <= 0) return TQ_EINVAL;
  if (rot->group != 32 && rot->group != 128) return TQ_EUNSUPPORTED;
  return TQ_OK;
}

tq_status check_cache(const tq_cache* c, const tq_rotation* rot, tq_role role) {
  if (c == nullptr || c->codes == nullptr || c->norms == nullptr) return TQ_EINVAL;
  if (c->role != role) return TQ_EINVAL;
  if (c->batch <= 0 || c->capacity <= 0 || (c->capacity % TQ_TILE) != 0) return TQ_EINVAL;
  // launch grid dimensions: the appends take (sequence, role) and KV heads as grid axes
  if (c->batch > 32767 || c->n_kv_heads > 65535) return TQ_EINVAL;
  if (c->n_kv_heads != rot->n_kv_heads) return TQ_EINVAL;
  if (c->group != rot->group) return TQ_EINVAL;
  if (c->bits != 3 && c->bits != 4) return TQ_EUNSUPPORTED;
  if (!valid_codebook(c->codebook, c->bits, c->group)) return TQ_EINVAL;
  if (c->capacity > TQ_MAX_CAPACITY) return TQ_ECAPACITY;
  return TQ_OK;
}

tq_status from_hip(hipError_t e) { return e == hipSuccess ? TQ_OK : TQ_EHIP; }

// Attention launches one workgroup per (row, KV head, section, head slice), at most one per
// (row, query head, section): that count must fit a one-dimensional grid.
bool grid_fits(int32_t batch, int32_t n_q_heads, int32_t n_splits) {
  // the counts are positive (checked before); the product of two fits 64 bits, the third divides
  return (int64_t)batch * n_q_heads <= INT32_MAX / n_splits;
}

// Host checks shared by the append calls; fills the launch arguments of one cache.
tq_status append_args(const tq_rotation* rot, const tq_cache* cache, const void* x, tq_dtype x_dtype, int32_t n_new,
                      const int32_t* pos, int32_t pos0, int32_t max_pos, tq::AppendArgs& a) {
  tq_status st = check_cache(cache, rot, cache ? cache->role : TQ_KEYS);
  if (st != TQ_OK) return st;
  if (cache->role != TQ_KEYS && cache->role != TQ_VALUES) return TQ_EINVAL;
  if (x == nullptr || n_new < 0) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_F16) return TQ_EINVAL;
  const int32_t first = pos ? max_pos : pos0;
  if (first < 0 || pos0 < 0) return TQ_EINVAL;
  if ((int64_t)first + n_new > cache->capacity) return TQ_ECAPACITY;
  std::memset(&a, 0, sizeof(a));
  a.x = x;
  a.codes = (uint8_t*)cache->codes;
  a.norms = cache->norms;
  a.signs = rot->signs;
  a.so4 = rot->so4;
  a.pos = pos;
  a.pos0 = pos0;
  a.n_new = n_new;
  a.n_kv_heads = cache->n_kv_heads;
  a.capacity = cache->capacity;
  for (int k = 0; k < 15; ++k) a.boundary[k] = cache->codebook.boundary[k];
  return TQ_OK;
}

// Tiles touched per (sequence, head): with a device-side start the alignment is unknown,
// so cover the worst case.
int append_tiles(const int32_t* pos, int32_t pos0, int32_t n_new) {
  const int span = pos ? (TQ_TILE - 1) + n_new : (pos0 % TQ_TILE) + n_new;
  return (span + TQ_TILE - 1) / TQ_TILE;
}

}  // namespace

extern "C" tq_status tq_quantize_append(const tq_rotation* rot, const tq_cache* cache, const void* x, tq_dtype x_dtype,
                                        int32_t n_new, const int32_t* pos, int32_t pos0, int32_t max_pos,
                                        void* stream) {
  tq_status st = check_rotation(rot);
  if (st != TQ_OK) return st;
  tq::AppendArgs a;
  if ((st = append_args(rot, cache, x, x_dtype, n_new, pos, pos0, max_pos, a)) != TQ_OK) return st;
  if (n_new == 0) return TQ_OK;
  return from_hip(tq::launch_append(a, cache->bits, cache->group, cache->role == TQ_VALUES, x_dtype == TQ_F16,
                                    cache->batch, append_tiles(pos, pos0, n_new), (hipStream_t)stream));
}

extern "C" tq_status tq_quantize_append_kv(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                           const void* xk, const void* xv, tq_dtype x_dtype, int32_t n_new,
                                           const int32_t* pos, int32_t pos0, int32_t max_pos, void* stream) {
  tq_status st = check_rotation(rot);
  if (st != TQ_OK) return st;
  if (keys == nullptr || values == nullptr) return TQ_EINVAL;
  if (keys->role != TQ_KEYS || values->role != TQ_VALUES) return TQ_EINVAL;
  if (keys->batch != values->batch) return TQ_EINVAL;
  tq::AppendArgs ak, av;
  if ((st = append_args(rot, keys, xk, x_dtype, n_new, pos, pos0, max_pos, ak)) != TQ_OK) return st;
  if ((st = append_args(rot, values, xv, x_dtype, n_new, pos, pos0, max_pos, av)) != TQ_OK) return st;
  if (n_new == 0) return TQ_OK;
  return from_hip(tq::launch_append_kv(ak, av, keys->bits, values->bits, keys->group, x_dtype == TQ_F16, keys->batch,
                                       append_tiles(pos, pos0, n_new), (hipStream_t)stream));
}

namespace {

// Host checks of a decode call; fills the launch arguments.  `same` reports whether keys and
// values share one four-code table (3-bit, identical codebooks).
tq_status decode_args(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values, const void* q,
                      tq_dtype q_dtype, int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                      int32_t n_splits, tq_schedule schedule, float* out, float* lse_out, float* part_o,
                      float* part_lse, tq::DecodeArgs& a, int& sched, bool& same) {
  tq_status st = check_rotation(rot);
  if (st != TQ_OK) return st;
  if ((st = check_cache(keys, rot, TQ_KEYS)) != TQ_OK) return st;
  if ((st = check_cache(values, rot, TQ_VALUES)) != TQ_OK) return st;
  if (keys->batch != values->batch) return TQ_EINVAL;
  if (q == nullptr || (q_dtype != TQ_F32 && q_dtype != TQ_F16)) return TQ_EINVAL;
  if (n_q_heads <= 0 || n_q_heads % rot->n_kv_heads != 0) return TQ_EINVAL;
  if (n_splits < 1 || max_len < 0 || !std::isfinite(scale)) return TQ_EINVAL;
  if (max_len > keys->capacity || max_len > values->capacity) return TQ_ECAPACITY;
  if (n_splits == 1 && out == nullptr) return TQ_EINVAL;
  if (n_splits > 1 && (part_o == nullptr || part_lse == nullptr)) return TQ_EINVAL;
  if (schedule != TQ_SCHEDULE_AUTO && schedule != TQ_SCHEDULE_VEC && schedule != TQ_SCHEDULE_MFMA) return TQ_EINVAL;
  if (values->capacity != keys->capacity) return TQ_EINVAL;

  const int group_size = n_q_heads / rot->n_kv_heads;
  if (!grid_fits(keys->batch, n_q_heads, n_splits)) return TQ_EINVAL;
  // every supported (bits, group) pair has a matrix-core kernel, and it is the faster schedule
  // at every cache length measured (32 to 8192 tokens, 1 to 8 query heads per KV head), so
  // AUTO takes it without a length threshold
  sched = schedule == TQ_SCHEDULE_VEC ? 1 : 2;

  std::memset(&a, 0, sizeof(a));
  a.kc = (const uint8_t*)keys->codes;
  a.kn = keys->norms;
  a.vc = (const uint8_t*)values->codes;
  a.vn = values->norms;
  a.q = q;
  a.seq_lens = seq_lens;
  a.signs = rot->signs;
  a.so4 = rot->so4;
  a.out = out;
  a.lse_out = lse_out;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.max_len = max_len;
  a.batch = keys->batch;
  a.n_kv_heads = rot->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group_size = group_size;
  const int hps = sched == 2 ? tq::mfma_heads_per_slice(rot->group) : 16;
  a.heads_per_slice = group_size < hps ? group_size : hps;
  a.n_slices = (group_size + a.heads_per_slice - 1) / a.heads_per_slice;
  a.n_splits = n_splits;
  a.capacity = keys->capacity;
  a.rot_group = rot->group;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kscale = keys->codebook.f16_scale;
  for (int k = 0; k < 16; ++k) {
    a.kcent[k] = keys->codebook.centroid[k];
    a.vcent[k] = values->codebook.centroid[k];
  }
  same = keys->bits == 3 && values->bits == 3 && keys->codebook.f16_scale == values->codebook.f16_scale;
  for (int k = 0; k < 8 && same; ++k) same = keys->codebook.centroid[k] == values->codebook.centroid[k];
  return TQ_OK;
}

}  // namespace

extern "C" tq_status tq_decode_attention(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                         const void* q, tq_dtype q_dtype, int32_t n_q_heads, const int32_t* seq_lens,
                                         int32_t max_len, float scale, int32_t n_splits, tq_schedule schedule,
                                         float* out, float* lse_out, float* part_o, float* part_lse, void* stream) {
  tq::DecodeArgs a;
  int sched;
  bool same;
  const tq_status st = decode_args(rot, keys, values, q, q_dtype, n_q_heads, seq_lens, max_len, scale, n_splits,
                                   schedule, out, lse_out, part_o, part_lse, a, sched, same);
  if (st != TQ_OK) return st;
  return from_hip(tq::launch_decode(a, sched, keys->bits, values->bits, q_dtype == TQ_F16, same, (hipStream_t)stream));
}

extern "C" tq_status tq_append_decode_attention(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                                const void* xk, const void* xv, tq_dtype x_dtype, const int32_t* pos,
                                                int32_t pos0, int32_t max_pos, const void* q, tq_dtype q_dtype,
                                                int32_t n_q_heads, float scale, int32_t n_splits,
                                                tq_schedule schedule, float* out, float* lse_out, float* part_o,
                                                float* part_lse, void* stream) {
  tq_status st = check_rotation(rot);
  if (st != TQ_OK) return st;
  if (keys == nullptr || values == nullptr) return TQ_EINVAL;
  if (keys->role != TQ_KEYS || values->role != TQ_VALUES) return TQ_EINVAL;
  if (keys->batch != values->batch) return TQ_EINVAL;
  tq::AppendArgs ak, av;
  if ((st = append_args(rot, keys, xk, x_dtype, 1, pos, pos0, max_pos, ak)) != TQ_OK) return st;
  if ((st = append_args(rot, values, xv, x_dtype, 1, pos, pos0, max_pos, av)) != TQ_OK) return st;
  // rows end at their new token: length pos[b] + 1, or pos0 + 1 for every row
  const int32_t max_len = (pos ? max_pos : pos0) + 1;
  tq::DecodeArgs a;
  int sched;
  bool same;
  if ((st = decode_args(rot, keys, values, q, q_dtype, n_q_heads, pos, max_len, scale, n_splits, schedule, out,
                        lse_out, part_o, part_lse, a, sched, same)) != TQ_OK)
    return st;
  a.len_bias = pos ? 1 : 0;
  const hipStream_t s = (hipStream_t)stream;
  if (sched == 1) {  // the vector schedule keeps two launches
    if ((st = from_hip(tq::launch_append_kv(ak, av, keys->bits, values->bits, keys->group, x_dtype == TQ_F16,
                                            keys->batch, append_tiles(pos, pos0, 1), s))) != TQ_OK)
      return st;
    return from_hip(tq::launch_decode(a, sched, keys->bits, values->bits, q_dtype == TQ_F16, same, s));
  }
  a.append = 1;
  a.append_f16 = x_dtype == TQ_F16;
  a.ak = ak;
  a.av = av;
  return from_hip(tq::launch_decode(a, sched, keys->bits, values->bits, q_dtype == TQ_F16, same, s));
}

extern "C" tq_status tq_append_decode_attention_static(const tq_rotation* rot, const tq_cache* keys,
                                                       const tq_cache* values, const void* xk, const void* xv,
                                                       tq_dtype x_dtype, const int32_t* pos, int32_t pos0,
                                                       int32_t max_pos, const void* q, tq_dtype q_dtype,
                                                       int32_t n_q_heads, float scale, int32_t n_splits,
                                                       tq_schedule schedule, float* out, float* lse_out,
                                                       void* stream) {
  if (out == nullptr || n_q_heads <= 0 || n_splits < 1 || keys == nullptr || keys->batch <= 0) return TQ_EINVAL;
  if (n_splits == 1)  // no partials: the step writes out itself
    return tq_append_decode_attention(rot, keys, values, xk, xv, x_dtype, pos, pos0, max_pos, q, q_dtype, n_q_heads,
                                      scale, 1, schedule, out, lse_out, nullptr, nullptr, stream);
  const int64_t rows = (int64_t)n_splits * keys->batch * n_q_heads;
  if (rows * (TQ_HEAD_DIM + 1) > tq::kStaticPartialFloats) return TQ_ECAPACITY;
  float* part = nullptr;
  if (tq::static_partials(&part) != hipSuccess) return TQ_EHIP;
  float* part_lse = part + rows * TQ_HEAD_DIM;
  const tq_status st = tq_append_decode_attention(rot, keys, values, xk, xv, x_dtype, pos, pos0, max_pos, q, q_dtype,
                                                  n_q_heads, scale, n_splits, schedule, nullptr, nullptr, part,
                                                  part_lse, stream);
  if (st != TQ_OK) return st;
  return tq_merge_splits(rot, n_splits, keys->batch, n_q_heads, part, part_lse, out, lse_out, stream);
}

extern "C" tq_status tq_dense_attention(const tq_rotation* rot, const void* k, const void* v, tq_dtype kv_dtype,
                                        int32_t batch, int32_t capacity, const void* q, tq_dtype q_dtype,
                                        int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                                        int32_t n_splits, float* part_o, float* part_lse, void* stream) {
  tq_status st = check_rotation(rot);
  if (st != TQ_OK) return st;
  if (k == nullptr || v == nullptr || q == nullptr || part_o == nullptr || part_lse == nullptr) return TQ_EINVAL;
  if ((kv_dtype != TQ_F32 && kv_dtype != TQ_F16) || (q_dtype != TQ_F32 && q_dtype != TQ_F16)) return TQ_EINVAL;
  if (batch <= 0 || capacity <= 0 || n_q_heads <= 0 || n_q_heads % rot->n_kv_heads != 0) return TQ_EINVAL;
  if (n_splits < 1 || max_len < 0 || !std::isfinite(scale)) return TQ_EINVAL;
  if (!grid_fits(batch, n_q_heads, n_splits)) return TQ_EINVAL;
  if (max_len > capacity) return TQ_ECAPACITY;
  if (capacity > TQ_MAX_CAPACITY) return TQ_ECAPACITY;  // 32-bit byte offsets within a stream's fp16 rows
  tq::DenseArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k = k;
  a.v = v;
  a.q = q;
  a.seq_lens = seq_lens;
  a.signs = rot->signs;
  a.so4 = rot->so4;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.max_len = max_len;
  a.batch = batch;
  a.n_kv_heads = rot->n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group_size = n_q_heads / rot->n_kv_heads;
  a.heads_per_slice = a.group_size < 8 ? a.group_size : 8;
  a.n_slices = (a.group_size + a.heads_per_slice - 1) / a.heads_per_slice;
  a.n_splits = n_splits;
  a.capacity = capacity;
  a.rot_group = rot->group;
  a.scale_log2 = scale * 1.4426950408889634f;
  return from_hip(tq::launch_dense(a, kv_dtype == TQ_F16, q_dtype == TQ_F16, (hipStream_t)stream));
}

extern "C" tq_status tq_merge_splits(const tq_rotation* rot, int32_t n_splits, int32_t batch, int32_t n_q_heads,
                                     const float* part_o, const float* part_lse, float* out, float* lse_out,
                                     void* stream) {
  if (rot != nullptr) {
    tq_status st = check_rotation(rot);
    if (st != TQ_OK) return st;
  }
  if (n_splits < 1 || batch <= 0 || n_q_heads <= 0) return TQ_EINVAL;
  if ((int64_t)batch * n_q_heads > INT32_MAX) return TQ_EINVAL;  // one thread group per output row
  if (rot != nullptr && n_q_heads % rot->n_kv_heads != 0) return TQ_EINVAL;
  if (part_o == nullptr || part_lse == nullptr || out == nullptr) return TQ_EINVAL;
  tq::MergeArgs a;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.out = out;
  a.lse_out = lse_out;
  // no rotation: partials of the original domain, merged without the inverse rotation
  a.signs = rot ? rot->signs : nullptr;
  a.so4 = rot ? rot->so4 : nullptr;
  a.n_splits = n_splits;
  a.batch = batch;
  a.n_q_heads = n_q_heads;
  a.group_size = rot ? n_q_heads / rot->n_kv_heads : 1;
  a.rot_group = rot ? rot->group : 128;
  return from_hip(tq::launch_merge(a, (hipStream_t)stream));
}

extern "C" tq_status tq_zip_compress(const void* x, tq_role role, int32_t batch, int32_t n_kv_heads, int32_t x_rows,
                                     int32_t src_page0, int32_t dst_page0, int32_t n_pages, uint8_t* store,
                                     uint8_t* meta, int32_t store_pages, void* stream) {
  if (x == nullptr || store == nullptr || meta == nullptr) return TQ_EINVAL;
  if (role != TQ_KEYS && role != TQ_VALUES) return TQ_EINVAL;
  if (batch <= 0 || n_kv_heads <= 0 || x_rows <= 0 || store_pages <= 0) return TQ_EINVAL;
  if (src_page0 < 0 || dst_page0 < 0 || n_pages < 0) return TQ_EINVAL;
  if ((int64_t)tq::kZipPage * ((int64_t)src_page0 + n_pages) > x_rows) return TQ_ECAPACITY;
  if ((int64_t)dst_page0 + n_pages > store_pages) return TQ_ECAPACITY;
  if ((int64_t)store_pages * tq::kZipSlot > 0xFFFFFFFFll) return TQ_ECAPACITY;  // 32-bit start offsets
  if (batch > 65535 || n_kv_heads > 65535) return TQ_EINVAL;                     // grid z and y
  if (n_pages == 0) return TQ_OK;
  tq::ZipCompressArgs a;
  a.x = (const uint16_t*)x;
  a.values = role == TQ_VALUES;
  a.store = store;
  a.meta = meta;
  a.n_kv_heads = n_kv_heads;
  a.x_rows = x_rows;
  a.store_pages = store_pages;
  a.src_page0 = src_page0;
  a.dst_page0 = dst_page0;
  return from_hip(tq::launch_zip_compress(a, batch, n_pages, (hipStream_t)stream));
}

extern "C" tq_status tq_zip_attention(const uint8_t* k_store, const uint8_t* k_meta, const uint8_t* v_store,
                                      const uint8_t* v_meta, int32_t store_pages, const void* k_tail,
                                      const void* v_tail, int32_t tail_rows, int32_t batch, int32_t n_kv_heads,
                                      const void* q, tq_dtype q_dtype, int32_t n_q_heads, const int32_t* seq_lens,
                                      int32_t max_len, float scale, int32_t n_splits, float* out, float* lse_out,
                                      float* part_o, float* part_lse, void* stream) {
  if (k_store == nullptr || k_meta == nullptr || v_store == nullptr || v_meta == nullptr) return TQ_EINVAL;
  if (k_tail == nullptr || v_tail == nullptr || q == nullptr) return TQ_EINVAL;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16 && q_dtype != TQ_BF16) return TQ_EINVAL;
  if (batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0) return TQ_EINVAL;
  if (store_pages < 0 || tail_rows <= 0 || tail_rows % tq::kZipPage != 0) return TQ_EINVAL;
  if (n_splits < 1 || max_len < 0 || !std::isfinite(scale)) return TQ_EINVAL;
  if (n_splits == 1 ? out == nullptr : (part_o == nullptr || part_lse == nullptr)) return TQ_EINVAL;
  const int group = n_q_heads / n_kv_heads;
  if (group > 8 && group % 8 != 0) return TQ_EINVAL;
  if ((int64_t)store_pages * tq::kZipSlot > 0xFFFFFFFFll) return TQ_ECAPACITY;
  if ((int64_t)max_len > (int64_t)tq::kZipPage * store_pages + tq::kZipPage - 1) return TQ_ECAPACITY;
  if (store_pages == 0 && max_len > tail_rows) return TQ_ECAPACITY;
  if (!grid_fits(batch, n_q_heads, n_splits)) return TQ_EINVAL;
  const int hps = group <= 4 ? group : 8;
  tq::ZipAttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.k_store = k_store;
  a.k_meta = k_meta;
  a.v_store = v_store;
  a.v_meta = v_meta;
  a.k_tail = (const uint16_t*)k_tail;
  a.v_tail = (const uint16_t*)v_tail;
  a.q = q;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse_out = lse_out;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.max_len = max_len;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group_size = group;
  a.heads_per_slice = hps;
  a.n_slices = (group + hps - 1) / hps;
  a.n_splits = n_splits;
  a.store_pages = store_pages;
  a.tail_rows = tail_rows;
  a.scale_log2 = scale * 1.4426950408889634f;
  return from_hip(tq::launch_zip_attention(a, (int)q_dtype, (hipStream_t)stream));
}

// A Block-GTQ record's code bytes: 64 (nibbles only) up to 128, a multiple of 16.
static bool valid_gtq_code_bytes(int32_t b) { return b >= 64 && b <= 128 && b % 16 == 0; }

static tq_status gtq_quantize(const tq_gtq_head* heads, const float* rotations, const float* proj, const void* x,
                              tq_dtype x_dtype, int32_t batch, int32_t n_kv_heads, int32_t n_new, int32_t pos0,
                              int32_t capacity, int32_t code_bytes, uint8_t* codes, float* norms, uint8_t* signs,
                              int32_t code_bits, void* stream) {
  if (heads == nullptr || rotations == nullptr || x == nullptr || codes == nullptr || norms == nullptr)
    return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (batch <= 0 || batch > 65535 || n_kv_heads <= 0 || n_kv_heads > 65535 || n_new < 0 || pos0 < 0 || capacity <= 0)
    return TQ_EINVAL;
  if (code_bits == 0 && !valid_gtq_code_bytes(code_bytes)) return TQ_EINVAL;
  if ((int64_t)pos0 + n_new > capacity || capacity > TQ_MAX_CAPACITY) return TQ_ECAPACITY;
  if (n_new == 0) return TQ_OK;
  tq::GtqQuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.heads = heads;
  a.rotations = rotations;
  a.x = x;
  a.codes = codes;
  a.norms = norms;
  a.n_kv_heads = n_kv_heads;
  a.n_new = n_new;
  a.pos0 = pos0;
  a.capacity = capacity;
  a.proj = proj;
  a.signs = signs;
  a.code_bits = code_bits;
  a.code_bytes = code_bits ? 16 * code_bits : code_bytes;
  return from_hip(tq::launch_gtq_quantize(a, x_dtype == TQ_F16, batch, (hipStream_t)stream));
}

extern "C" tq_status tq_gtq_quantize_keys(const tq_gtq_head* heads, const float* rotations, const void* x,
                                          tq_dtype x_dtype, int32_t batch, int32_t n_kv_heads, int32_t n_new,
                                          int32_t pos0, int32_t capacity, int32_t code_bytes, uint8_t* codes,
                                          float* norms, void* stream) {
  return gtq_quantize(heads, rotations, nullptr, x, x_dtype, batch, n_kv_heads, n_new, pos0, capacity, code_bytes,
                      codes, norms, nullptr, 0, stream);
}

extern "C" tq_status tq_gtq_qjl_quantize_keys(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                              int32_t mse_bits, const void* x, tq_dtype x_dtype, int32_t batch, int32_t n_kv_heads,
                                              int32_t n_new, int32_t pos0, int32_t capacity, uint8_t* codes,
                                              float* norms, uint8_t* signs, void* stream) {
  if (proj == nullptr || signs == nullptr || mse_bits < 1 || mse_bits > 3) return TQ_EINVAL;
  return gtq_quantize(heads, rotations, proj, x, x_dtype, batch, n_kv_heads, n_new, pos0, capacity, 0, codes, norms,
                      signs, mse_bits, stream);
}

static tq_status gtq_attention_args(const tq_gtq_head* heads, const float* rotations, int32_t code_bytes,
                                    const uint8_t* codes,
                                    const float* norms, const void* v, int32_t capacity, int32_t batch,
                                    int32_t n_kv_heads, const void* q, tq_dtype q_dtype, int32_t n_q_heads,
                                    const int32_t* seq_lens, int32_t max_len, float scale, int32_t n_splits,
                                    float* out, float* lse_out, float* part_o, float* part_lse, tq::GtqAttnArgs& a) {
  if (heads == nullptr || rotations == nullptr || codes == nullptr || norms == nullptr || v == nullptr || q == nullptr)
    return TQ_EINVAL;
  if (q_dtype != TQ_F32 && q_dtype != TQ_F16) return TQ_EINVAL;
  if (batch <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads != 0 || capacity <= 0)
    return TQ_EINVAL;
  if (n_splits < 1 || max_len < 0 || !std::isfinite(scale)) return TQ_EINVAL;
  if (!grid_fits(batch, n_q_heads, n_splits)) return TQ_EINVAL;
  if (n_splits == 1 ? out == nullptr : (part_o == nullptr || part_lse == nullptr)) return TQ_EINVAL;
  if (code_bytes != 0 && !valid_gtq_code_bytes(code_bytes)) return TQ_EINVAL;
  if (max_len > capacity) return TQ_ECAPACITY;
  if (capacity > TQ_MAX_CAPACITY) return TQ_ECAPACITY;  // 32-bit byte offsets within a stream's values
  const int group = n_q_heads / n_kv_heads;
  const int hps = group < 8 ? group : 8;
  const int slices = (group + hps - 1) / hps;
  if ((int64_t)batch * n_kv_heads * n_splits * slices > 0x7FFFFFFFll) return TQ_EINVAL;
  std::memset(&a, 0, sizeof(a));
  a.heads = heads;
  a.rotations = rotations;
  a.codes = codes;
  a.norms = norms;
  a.v = v;
  a.q = q;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse_out = lse_out;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.max_len = max_len;
  a.batch = batch;
  a.n_kv_heads = n_kv_heads;
  a.n_q_heads = n_q_heads;
  a.group_size = group;
  a.heads_per_slice = hps;
  a.n_slices = slices;
  a.n_splits = n_splits;
  a.capacity = capacity;
  a.code_bytes = code_bytes;
  a.scale_log2 = scale * 1.4426950408889634f;
  return TQ_OK;
}

extern "C" tq_status tq_gtq_attention(const tq_gtq_head* heads, const float* rotations, int32_t code_bytes,
                                      const uint8_t* codes,
                                      const float* norms, const void* v, int32_t capacity, int32_t batch,
                                      int32_t n_kv_heads, const void* q, tq_dtype q_dtype, int32_t n_q_heads,
                                      const int32_t* seq_lens, int32_t max_len, float scale, int32_t n_splits,
                                      float* out, float* lse_out, float* part_o, float* part_lse, void* stream) {
  if (!valid_gtq_code_bytes(code_bytes)) return TQ_EINVAL;
  tq::GtqAttnArgs a;
  const tq_status st = gtq_attention_args(heads, rotations, code_bytes, codes, norms, v, capacity, batch, n_kv_heads, q, q_dtype,
                                          n_q_heads, seq_lens, max_len, scale, n_splits, out, lse_out, part_o,
                                          part_lse, a);
  if (st != TQ_OK) return st;
  return from_hip(tq::launch_gtq_attention(a, q_dtype == TQ_F16, (hipStream_t)stream));
}

extern "C" tq_status tq_gtq_qjl_attention(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                          int32_t mse_bits, const uint8_t* codes, const float* norms, const uint8_t* signs, const void* v,
                                          int32_t capacity, int32_t batch, int32_t n_kv_heads, const void* q,
                                          tq_dtype q_dtype, int32_t n_q_heads, const int32_t* seq_lens,
                                          int32_t max_len, float scale, int32_t n_splits, float* out, float* lse_out,
                                          float* part_o, float* part_lse, void* stream) {
  if (proj == nullptr || signs == nullptr || mse_bits < 1 || mse_bits > 3) return TQ_EINVAL;
  tq::GtqAttnArgs a;
  const tq_status st = gtq_attention_args(heads, rotations, 0, codes, norms, v, capacity, batch, n_kv_heads, q, q_dtype,
                                          n_q_heads, seq_lens, max_len, scale, n_splits, out, lse_out, part_o,
                                          part_lse, a);
  if (st != TQ_OK) return st;
  a.proj = proj;
  a.signs = signs;
  a.code_bits = mse_bits;
  return from_hip(tq::launch_gtq_attention(a, q_dtype == TQ_F16, (hipStream_t)stream));
}

static tq_status gtq_append_step(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                 int32_t code_bits, int32_t code_bytes, uint8_t* codes, float* norms, uint8_t* signs, void* v, int32_t capacity,
                                 int32_t batch, int32_t n_kv_heads, const void* k_new, const void* v_new,
                                 tq_dtype x_dtype, const int32_t* pos, int32_t pos0, int32_t max_pos, const void* q,
                                 tq_dtype q_dtype, int32_t n_q_heads, float scale, int32_t n_splits, float* out,
                                 float* lse_out, float* part_o, float* part_lse, void* stream) {
  if (k_new == nullptr || v_new == nullptr) return TQ_EINVAL;
  if (x_dtype != TQ_F32 && x_dtype != TQ_F16) return TQ_EINVAL;
  if (pos0 < 0 || (pos != nullptr && max_pos < 0)) return TQ_EINVAL;
  // rows end at their new token: length pos[b] + 1, or pos0 + 1 for every row
  const int64_t max_len = (int64_t)(pos ? max_pos : pos0) + 1;
  if (max_len > capacity) return TQ_ECAPACITY;
  tq::GtqAttnArgs a;
  const tq_status st = gtq_attention_args(heads, rotations, code_bytes, codes, norms, v, capacity, batch, n_kv_heads, q, q_dtype,
                                          n_q_heads, pos, (int32_t)max_len, scale, n_splits, out, lse_out, part_o,
                                          part_lse, a);
  if (st != TQ_OK) return st;
  a.append = 1;
  a.x_f16 = x_dtype == TQ_F16;
  a.len_bias = pos ? 1 : 0;
  a.k_new = k_new;
  a.v_new = v_new;
  a.w_codes = codes;
  a.w_norms = norms;
  a.w_v = v;
  a.proj = proj;
  a.signs = signs;
  a.w_signs = signs;
  a.code_bits = code_bits;
  return from_hip(tq::launch_gtq_attention(a, q_dtype == TQ_F16, (hipStream_t)stream));
}

extern "C" tq_status tq_gtq_append_attention(const tq_gtq_head* heads, const float* rotations, int32_t code_bytes,
                                             uint8_t* codes,
                                             float* norms, void* v, int32_t capacity, int32_t batch,
                                             int32_t n_kv_heads, const void* k_new, const void* v_new,
                                             tq_dtype x_dtype, const int32_t* pos, int32_t pos0, int32_t max_pos,
                                             const void* q, tq_dtype q_dtype, int32_t n_q_heads, float scale,
                                             int32_t n_splits, float* out, float* lse_out, float* part_o,
                                             float* part_lse, void* stream) {
  if (!valid_gtq_code_bytes(code_bytes)) return TQ_EINVAL;
  return gtq_append_step(heads, rotations, nullptr, 0, code_bytes, codes, norms, nullptr, v, capacity, batch, n_kv_heads, k_new,
                         v_new, x_dtype, pos, pos0, max_pos, q, q_dtype, n_q_heads, scale, n_splits, out, lse_out,
                         part_o, part_lse, stream);
}

extern "C" tq_status tq_gtq_qjl_append_attention(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                                 int32_t mse_bits, uint8_t* codes, float* norms, uint8_t* signs, void* v,
                                                 int32_t capacity, int32_t batch, int32_t n_kv_heads,
                                                 const void* k_new, const void* v_new, tq_dtype x_dtype,
                                                 const int32_t* pos, int32_t pos0, int32_t max_pos, const void* q,
                                                 tq_dtype q_dtype, int32_t n_q_heads, float scale, int32_t n_splits,
                                                 float* out, float* lse_out, float* part_o, float* part_lse,
                                                 void* stream) {
  if (proj == nullptr || signs == nullptr || mse_bits < 1 || mse_bits > 3) return TQ_EINVAL;
  return gtq_append_step(heads, rotations, proj, mse_bits, 0, codes, norms, signs, v, capacity, batch, n_kv_heads, k_new, v_new,
                         x_dtype, pos, pos0, max_pos, q, q_dtype, n_q_heads, scale, n_splits, out, lse_out, part_o,
                         part_lse, stream);
}

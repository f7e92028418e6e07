// Launch-level interface between the C ABI (tq_api.cpp) and the HIP kernels
// (tq_kernels.hip).  Plain structs passed by value as kernel arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kHeadDim = 128;
constexpr int kTile = 32;

struct AppendArgs {
  const void* x;            // [batch][n_kv_heads][n_new][128]
  uint8_t* codes;
  float* norms;
  const float* signs;       // [n_kv_heads][128]
  const float* so4;         // [n_kv_heads][32][2][4] or null
  const int32_t* pos;       // [batch] or null
  int32_t pos0;
  int32_t n_new;
  int32_t n_kv_heads;
  int32_t capacity;
  float boundary[15];
  // edge mode of the tile kernel: when n_edges > 0, block x handles tile edge[x] (tiles
  // counted from pos / 32) and nothing else; the whole tiles between went to the
  // matrix-core append
  int32_t n_edges;
  int32_t edge[2];
};

struct DecodeArgs {
  const uint8_t* kc;        // key records
  const float* kn;          // key norms
  const uint8_t* vc;        // value tiles
  const float* vn;          // value norms
  const void* q;            // [batch][n_q_heads][128]
  const int32_t* seq_lens;  // [batch] or null
  const float* signs;
  const float* so4;
  float* out;               // n_splits == 1
  float* lse_out;           // optional
  float* part_o;            // n_splits > 1
  float* part_lse;
  int32_t max_len;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group_size;       // query heads per KV head
  int32_t heads_per_slice;  // query heads one workgroup serves
  int32_t n_slices;         // workgroups per (sequence, KV head, split)
  int32_t n_splits;
  int32_t capacity;
  int32_t rot_group;        // 32 or 128
  float scale_log2;         // softmax scale * log2(e)
  float kscale;             // key codebook scale making every level nearly fp16-exact (also
                            // the value scale when keys and values share one table)
  float kcent[16];
  float vcent[16];
  // Fused single-token append: the workgroups whose section holds a row's new position
  // quantise and write that token (keys and values) before reading the cache.
  int32_t append;           // 0 or 1
  int32_t append_f16;       // the new vectors are fp16
  int32_t len_bias;         // a row has seq_lens[b] + len_bias tokens (1: seq_lens holds positions)
  AppendArgs ak, av;
};

// Attention over an unquantised (fp16/fp32) K/V region, written as key-axis section partials
// in the rotated domain so that they merge with the packed sections.
struct DenseArgs {
  const void* k;            // [batch][n_kv_heads][capacity][128]
  const void* v;
  const void* q;            // [batch][n_q_heads][128]
  const int32_t* seq_lens;  // [batch] or null
  const float* signs;
  const float* so4;
  float* part_o;            // [n_splits][batch][n_q_heads][128]
  float* part_lse;          // [n_splits][batch][n_q_heads]
  int32_t max_len;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group_size;
  int32_t heads_per_slice;
  int32_t n_slices;
  int32_t n_splits;
  int32_t capacity;
  int32_t rot_group;
  float scale_log2;
};

// Lossless BF16 exponent codec of a KV cache (16-token pages, 4096-byte page slots, 8
// bytes of metadata per page) and attention read straight from it.
constexpr int kZipPage = 16;
constexpr int kZipSlot = 4096;

struct ZipCompressArgs {
  const uint16_t* x;   // BF16 [batch][n_kv_heads][x_rows][128]
  int32_t values;      // 0 keys (chunks of 4 tokens), 1 values (chunks of 32 coordinates)
  uint8_t* store;      // [batch][n_kv_heads][store_pages][4096]
  uint8_t* meta;       // [batch][n_kv_heads][store_pages][8]
  int32_t n_kv_heads;
  int32_t x_rows;
  int32_t store_pages;
  int32_t src_page0;   // page i of the call reads x rows 16 (src_page0 + i) ..
  int32_t dst_page0;   // .. and becomes store page dst_page0 + i
};

struct ZipAttnArgs {
  const uint8_t* k_store;  // as ZipCompressArgs
  const uint8_t* k_meta;
  const uint8_t* v_store;
  const uint8_t* v_meta;
  const uint16_t* k_tail;  // BF16 [batch][n_kv_heads][tail_rows][128]: tokens past the last full page
  const uint16_t* v_tail;
  const void* q;           // [batch][n_q_heads][128]
  const int32_t* seq_lens; // [batch] or null
  float* out;              // n_splits == 1: [batch][n_q_heads][128]
  float* lse_out;          // optional
  float* part_o;           // n_splits > 1: [n_splits][batch][n_q_heads][128]
  float* part_lse;         // [n_splits][batch][n_q_heads]
  int32_t max_len;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group_size;
  int32_t heads_per_slice;
  int32_t n_slices;
  int32_t n_splits;
  int32_t store_pages;
  int32_t tail_rows;
  float scale_log2;
};

// Block-GTQ keys (heads: tq_gtq_head layout, declared in tq.h).
struct GtqQuantArgs {
  const void* heads;        // tq_gtq_head [n_kv_heads]
  const float* rotations;   // [n_kv_heads][16384]
  const void* x;            // [batch][n_kv_heads][n_new][128]
  uint8_t* codes;           // [batch][n_kv_heads][capacity][code_bytes, or 16 code_bits]
  float* norms;             // [batch][n_kv_heads][capacity][4]
  int32_t n_kv_heads;
  int32_t n_new;
  int32_t pos0;
  int32_t capacity;
  const float* proj;        // two-stage keys: [n_kv_heads][128][128], (S Q)^T; else NULL
  uint8_t* signs;           // two-stage keys: [batch][n_kv_heads][capacity][16]; else NULL
  int32_t code_bits;        // 0: Block-GTQ records, codes [..][code_bytes]; 1-3: two-stage keys'
                            // first stage bit-packed at that width, codes [..][16 code_bits]
  int32_t code_bytes;       // Block-GTQ record code bytes: 64 .. 128, a multiple of 16
};

struct GtqAttnArgs {
  const void* heads;
  const float* rotations;
  const uint8_t* codes;
  const float* norms;
  const void* v;            // fp16 [batch][n_kv_heads][capacity][128]
  const void* q;
  const int32_t* seq_lens;
  float* out;
  float* lse_out;
  float* part_o;
  float* part_lse;
  int32_t max_len;
  int32_t batch;
  int32_t n_kv_heads;
  int32_t n_q_heads;
  int32_t group_size;
  int32_t heads_per_slice;
  int32_t n_slices;
  int32_t n_splits;
  int32_t capacity;
  float scale_log2;
  // Fused append (append != 0): each row's new key is encoded and its value row written at
  // slot seq_lens[b] (or max_len - 1 when seq_lens is NULL) before the section holding that
  // slot reads the cache; rows then end there (len_bias = 1: length seq_lens[b] + 1).
  int32_t append;
  int32_t x_f16;            // k_new and v_new are fp16 (else fp32; values stored as fp16)
  int32_t len_bias;
  const void* k_new;        // [batch][n_kv_heads][128]
  const void* v_new;        // [batch][n_kv_heads][128]
  uint8_t* w_codes;         // the cache again, writable (append only)
  float* w_norms;
  void* w_v;
  // two-stage keys (signs != NULL): proj [n_kv_heads][128][128] = (S Q)^T, signs
  // [batch][n_kv_heads][capacity][16]
  const float* proj;
  const uint8_t* signs;
  uint8_t* w_signs;         // writable, for the fused append of two-stage keys
  int32_t code_bits;        // 0: Block-GTQ records, codes [..][code_bytes]; 1-3: two-stage keys'
                            // first stage bit-packed at that width, codes [..][16 code_bits]
  int32_t code_bytes;       // Block-GTQ record code bytes: 64 .. 128, a multiple of 16
};

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  float* out;
  float* lse_out;
  const float* signs;
  const float* so4;
  int32_t n_splits;
  int32_t batch;
  int32_t n_q_heads;
  int32_t group_size;
  int32_t rot_group;
};

// Each returns the hipError_t of the launch.
hipError_t launch_append(const AppendArgs& a, int bits, int group, bool values, bool x_f16, int batch,
                         int n_tiles, hipStream_t stream);
// Keys and values in one launch (both caches share batch, heads, group and rotation).
hipError_t launch_append_kv(const AppendArgs& ak, const AppendArgs& av, int bits_k, int bits_v, int group, bool x_f16,
                            int batch, int n_tiles, hipStream_t stream);
// schedule: 1 = vector (fp32), 2 = matrix cores
// shared_table: 3-bit keys and values with identical codebooks (one four-code table)
hipError_t launch_decode(const DecodeArgs& a, int schedule, int bits_k, int bits_v, bool q_f16, bool shared_table,
                         hipStream_t stream);
hipError_t launch_dense(const DenseArgs& a, bool kv_f16, bool q_f16, hipStream_t stream);
hipError_t launch_dense_mfma(const DenseArgs& a, bool q_f16, hipStream_t stream);  // fp16 K/V (tq_dense.hip)
hipError_t launch_zip_compress(const ZipCompressArgs& a, int batch, int n_pages, hipStream_t stream);
// q_type: 0 fp32, 1 fp16, 2 bf16
hipError_t launch_zip_attention(const ZipAttnArgs& a, int q_type, hipStream_t stream);
hipError_t launch_gtq_quantize(const GtqQuantArgs& a, bool x_f16, int batch, hipStream_t stream);
hipError_t launch_gtq_attention(const GtqAttnArgs& a, bool q_f16, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);

// Library-owned device buffer for the section partials of the allocation-free decode step:
// kStaticPartialFloats floats per device (4 MiB), shared by every call on that device.  Sets
// *p to the calling thread's current device's copy (its address is looked up once per
// device); returns the hipError_t of the lookup.
constexpr int64_t kStaticPartialFloats = 1 << 20;
hipError_t static_partials(float** p);

// Heads one workgroup of the matrix-core schedule can serve: the 16 MFMA columns hold
// (norm group, head) pairs for 32-groups and (query part, head) pairs for whole-head groups.
inline int mfma_heads_per_slice(int rot_group) { return rot_group == 32 ? 4 : 8; }

}  // namespace tq

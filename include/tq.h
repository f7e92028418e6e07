/*
 * tq.h -- decode attention computed directly on a rotated, Lloyd-Max-quantised,
 * bit-packed KV cache (3- or 4-bit codes), for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Every pointer marked "device" is device memory owned by the caller; the library
 * never allocates or frees memory and launches everything on the HIP stream it is given
 * (passed as void* = hipStream_t, NULL = default stream).  Its only state: each device's
 * compute-unit count, read once (a thread-safe cache), and the static partial buffer of
 * tq_append_decode_attention_static with its per-device address.  Calls
 * return without synchronising.  Argument errors are detected on the host before any
 * launch: the call then returns TQ_EINVAL / TQ_EUNSUPPORTED / TQ_ECAPACITY and writes
 * nothing.  A failed launch returns TQ_EHIP.  No C++ exception crosses this boundary.
 *
 * The method (citations name the page and the section on it):
 *   * a key or value vector is split into groups of g coordinates (g = 32, or g = 128 =
 *     the whole head); each group stores its L2 norm, is divided by it and rotated
 *     ("TurboQuant: ... MNN on phones", 2.1 and 3.1);
 *   * the rotation is R = S_SO4 . H . D_s: per-coordinate +-1 sign flips, the normalised
 *     Walsh-Hadamard transform on every g-block (3.1), and optionally (IsoQuant) the
 *     SO(4) rotation v -> q_L v conj(q_R) of every 4-block ("RotaryQuant: Fitting 120B
 *     MoE Models ... Fused Compressed-Space Attention", key design 2);
 *   * every rotated coordinate is replaced by the index of its Lloyd-Max cell for the
 *     law f(t) ~ (1 - t^2)^((g-3)/2) ("TurboQuant ...", 2.2 and 2.3), the index being the
 *     number of cell boundaries strictly below the value (3.4);
 *   * decode rotates the query once, forms scores and the value sum in the rotated
 *     domain straight from the codes, and applies one inverse rotation to the output
 *     ("RotaryQuant ...", key design 3; "TurboQuant ...", 3.3);
 *   * long rows are split along the key axis and the partial results merged by
 *     log-sum-exp ("RoPE-Aware Bit Allocation for KV-Cache Quantization", packed-cache
 *     implementation details).
 *
 * Fixed sizes: head dimension 128; cache capacity a multiple of the 32-token tile and at
 * most TQ_MAX_CAPACITY tokens per (sequence, head) (packed, unquantised, Block-GTQ and
 * two-stage caches; the lossless page store states its own limits).
 *
 * Packed layout (the pages fix only the unit: 8 three-bit codes in 3 bytes, or two
 * four-bit codes per byte, "TurboQuant ...", 3.3).  A word of 8 codes of b bits is the
 * integer sum_j code_j << (b*j) stored little-endian in b bytes (3 or 4).
 *   keys:   codes [batch][n_kv_heads][capacity][16*b] bytes: per token 16 words, word w =
 *           coordinates 8w..8w+7 of that token.
 *   values: codes [batch][n_kv_heads][capacity/32][32*16*b] bytes: per 32-token tile 512
 *           words, word (q*16 + m)*8 + u = coordinate 16u + m of tile tokens
 *           16h + 4q + r (h = 0..1, r = 0..3) in slot 4h + r.
 *   norms (both): fp32 [batch][n_kv_heads][capacity/32][128/g][32]; tile token t is at
 *           position 8*((t >> 2) & 3) + 4*(t >> 4) + (t & 3).
 * Keys keep a token's coordinates together because scores contract over coordinates;
 * values keep 8 tokens of one coordinate together because the value sum contracts over
 * tokens.  Each is then one matrix-core operand row per word.
 */
#ifndef TQ_H
#define TQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_HEAD_DIM 128
#define TQ_TILE 32
/* Tokens per (sequence, head) of any cache: byte offsets within one stream stay 32-bit. */
#define TQ_MAX_CAPACITY (1 << 24)

/* Every enum below ends with a *_MAX_ENUM member: it gives the type the range of a 32-bit
 * int, so that any value a caller passes (an invalid one included, which the calls reject
 * with TQ_EINVAL) is a defined value of the type. */
typedef enum {
  TQ_OK = 0,
  TQ_EINVAL = 1,        /* null pointer, bad size or inconsistent arguments */
  TQ_EUNSUPPORTED = 2,  /* valid but not implemented (bits, group, head grouping) */
  TQ_ECAPACITY = 3,     /* a write or read would pass the cache capacity, or a capacity above TQ_MAX_CAPACITY */
  TQ_EHIP = 4,          /* a HIP launch or runtime call failed */
  TQ_STATUS_MAX_ENUM = 0x7FFFFFFF
} tq_status;

/* TQ_BF16 is accepted only where a declaration says so (the compressed BF16 cache). */
typedef enum { TQ_F32 = 0, TQ_F16 = 1, TQ_BF16 = 2, TQ_DTYPE_MAX_ENUM = 0x7FFFFFFF } tq_dtype;
typedef enum { TQ_KEYS = 0, TQ_VALUES = 1, TQ_ROLE_MAX_ENUM = 0x7FFFFFFF } tq_role;

/* Decode schedules.  MFMA: scores and value sum as matrix-core products of fp16
 * operands with fp32 accumulation (the key codebook scaled to be nearly fp16-exact, see
 * tq_codebook.f16_scale, and the query split into two fp16 parts).  VEC: plain fp32 vector arithmetic, token-parallel
 * scores and dimension-parallel value sum.  AUTO picks MFMA: measured on MI355X it is faster at
 * every cache length from 32 to 8192 tokens, for 1, 4 and 8 query heads per KV head and both
 * rotation groups (2x at 32 tokens, growing to 28-48x at 8192), so no length threshold applies. */
typedef enum {
  TQ_SCHEDULE_AUTO = 0,
  TQ_SCHEDULE_VEC = 1,
  TQ_SCHEDULE_MFMA = 2,
  TQ_SCHEDULE_MAX_ENUM = 0x7FFFFFFF
} tq_schedule;

/* Static description of an error code (never NULL). */
const char* tq_status_string(tq_status s);

/* Lloyd-Max codebook for one coordinate of a uniformly rotated unit vector in R^dim.
 * ("TurboQuant ...", 2.2: density f(t) ~ (1 - t^2)^((dim-3)/2) on [-1, 1];
 *  2.3: centroid = conditional mean of its cell, boundary = midpoint, iterate.)
 * Computed on the host in double precision (Gauss-Legendre quadrature of the cell
 * masses, closed-form first moments; in two dimensions, the arcsine law, closed-form
 * masses too) and stored rounded to float.
 * centroid[0 .. 2^bits-1] ascending; boundary[k] = (centroid[k] + centroid[k+1]) / 2 for
 * k < 2^bits - 1; unused entries are 0.  f16_scale is the s in [1, 2) (searched on a 2^-16
 * grid) at which every s * centroid[k] is nearest to an fp16 number in relative terms
 * (worst level: 2.6e-5 for 3-bit, 9e-5 for 4-bit codebooks of the supported groups, against
 * up to 3.2e-4 at s = 1); the matrix-core decode holds the key codebook as fp16(s * c) and
 * divides the query by s.  Host-only; no device work.
 * Errors: TQ_EINVAL if out == NULL; TQ_EUNSUPPORTED unless 1 <= bits <= 4 and dim >= 2
 * (the packed caches take 3 or 4 bits; Block-GTQ key groups take 1 to 4 bits and any even
 * dimension). */
typedef struct {
  int32_t bits;
  int32_t dim;
  float centroid[16];
  float boundary[15];
  float f16_scale;
} tq_codebook;

tq_status tq_make_codebook(int32_t bits, int32_t dim, tq_codebook* out);

/* Rotation shared by the keys, the values and the queries of one KV head. */
typedef struct {
  int32_t group;        /* g: Hadamard block = norm group = codebook dim; 32 or 128 */
  int32_t n_kv_heads;
  const float* signs;   /* device [n_kv_heads][128], each +1.0f or -1.0f, applied first */
  const float* so4;     /* device [n_kv_heads][32][2][4] unit quaternions (q_L, q_R) as
                           (real, i, j, k) for the 4-blocks, applied after the Hadamard;
                           NULL = no SO(4) stage */
} tq_rotation;

/* One packed tensor (keys or values) of a batch of sequences.  Caller-owned memory. */
typedef struct {
  void* codes;          /* device, layout above for `role` */
  float* norms;         /* device, layout above */
  int32_t batch;        /* 1 .. 32767 */
  int32_t n_kv_heads;   /* 1 .. 65535, the rotation's */
  int32_t capacity;     /* tokens per (sequence, head); multiple of 32, <= TQ_MAX_CAPACITY */
  int32_t bits;         /* 3 or 4 */
  int32_t group;        /* must equal the rotation's group */
  tq_role role;
  tq_codebook codebook; /* tq_make_codebook(bits, group) */
} tq_cache;

/* Quantise n_new new vectors per (sequence, KV head) into the cache: per group, norm ->
 * divide -> rotate -> codebook search -> pack ("TurboQuant ...", 2.1 and 3.3: quantise
 * on write, no intermediate fp16 copy).  One call handles a decode step (n_new = 1) or
 * a whole prompt (n_new = T; "RoPE-Aware Bit Allocation ...": one call per layer).
 *   x:     device [batch][n_kv_heads][n_new][128] of x_dtype, read only.
 *   pos:   device int32 [batch], first slot written per sequence, or NULL to use pos0
 *          for every sequence.  max_pos: host upper bound on pos[] used for the
 *          capacity check (ignored when pos == NULL).
 * Slots [pos, pos + n_new) of every (sequence, head) are written; neighbouring value
 * slots that share a packed word are preserved.  A zero group stores norm 0 and the
 * code of 0.  Errors: TQ_ECAPACITY if max(pos) + n_new > capacity or capacity >
 * TQ_MAX_CAPACITY. */
tq_status tq_quantize_append(const tq_rotation* rot, const tq_cache* cache, const void* x,
                             tq_dtype x_dtype, int32_t n_new, const int32_t* pos, int32_t pos0,
                             int32_t max_pos, void* stream);

/* The keys and the values of one step in one launch: the same result, bit for bit, as
 * tq_quantize_append(keys, xk) followed by tq_quantize_append(values, xv) with the same
 * n_new, pos, pos0 and max_pos ("TurboQuant ...", 3.3: K and V are quantised on write).
 * keys must have role TQ_KEYS and values TQ_VALUES, with equal batch; xk and xv are
 * device [batch][n_kv_heads][n_new][128] of x_dtype.  Errors as tq_quantize_append,
 * checked for both caches before anything is launched. */
tq_status tq_quantize_append_kv(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                const void* xk, const void* xv, tq_dtype x_dtype, int32_t n_new,
                                const int32_t* pos, int32_t pos0, int32_t max_pos, void* stream);

/* One decode step of attention for every query head against the packed cache, computed
 * in the rotated domain straight from the codes: the query is rotated once per head, each
 * score is the sum over groups of the key group norm times the dot of the rotated query with
 * the codebook values of the key's codes, the value sum accumulates the weight times the
 * value group norm times the value's codebook values, and one inverse rotation is applied to
 * the output ("TurboQuant: ... MNN on phones", 3.3, the key and value paths;
 * "RotaryQuant ...", key design 3: score, softmax, value accumulation and inverse rotation
 * fused over the packed cache; "RoPE-Aware Bit Allocation ...", packed-cache implementation
 * details: the key axis split into sections merged by log-sum-exp).
 *   q:        device [batch][n_q_heads][128] of q_dtype; query head h reads KV head
 *             h / (n_q_heads / n_kv_heads) (contiguous groups).
 *   seq_lens: device int32 [batch] (each <= max_len) or NULL = every row has max_len
 *             tokens; max_len <= capacity.
 *   scale:    softmax scale applied to q.k (1/sqrt(128) in the usual convention).
 *   n_splits: key-axis sections; section s of a length-T row covers tokens
 *             [s*C, min(T, (s+1)*C)), C = ceil(T / n_splits).
 * n_splits == 1: writes out [batch][n_q_heads][128] fp32 (original domain) and, if not
 *             NULL, lse_out [batch][n_q_heads] (natural log of the softmax denominator).
 * n_splits > 1: writes part_o [n_splits][batch][n_q_heads][128] (rotated domain,
 *             normalised per section) and part_lse [n_splits][batch][n_q_heads]; an empty
 *             section has lse = -inf and a zero partial.  Finish with tq_merge_splits.
 * A row with no tokens gives out = 0 and lse = -inf.
 * The MFMA schedule converts the scaled query (after an exact power-of-two prescale, split
 * into fp16 high and low parts) and the value weights p * value-norm to fp16, and holds the
 * codebook levels as fp16 at their fp16-exact scale (worst level 2.6e-5 for 3-bit, 9e-5 for
 * 4-bit codebooks).  The value weights carry a power of two that is reset per 32-token block
 * whenever a weight would pass 2^15 or all of the block's weights fall below 2^-10 (the sum
 * of the weights carries it too, so it cancels): any value norm up to about 2^100 keeps the
 * weights in fp16's range, and each block's largest weights at full fp16 precision.  Scores
 * carry the codebook's level error, at most that relative error times scale * |q| * |k|:
 * on keys and queries with 8x outlier channels (scores up to about 30) lse errors up to
 * 9e-4 were measured with 3-bit keys and 1.7e-3 with 4-bit keys, and output rows up to
 * 1.3e-3 off; with two 10x channels shared by queries and keys (scores near 90) output rows
 * reach 2-3e-3.  For such inputs the VEC schedule (fp32 levels) keeps rows near 1e-5.  When an output row is carried by a token far below the softmax maximum
 * (weight 1e-6 but a value norm 1e4 times the others), that absolute score error becomes the
 * row's relative error.  The VEC schedule is fp32 throughout.
 * Errors: TQ_EINVAL for null pointers, bad dtypes, counts (batch * n_q_heads * n_splits at
 * most 2^31 - 1), scale or schedule, caches that do not match the rotation or each other, or
 * a missing output for the split count;
 * TQ_ECAPACITY for max_len > capacity or capacity > TQ_MAX_CAPACITY; TQ_EUNSUPPORTED for
 * bits or groups outside 3/4 and 32/128. */
tq_status tq_decode_attention(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                              const void* q, tq_dtype q_dtype, int32_t n_q_heads,
                              const int32_t* seq_lens, int32_t max_len, float scale,
                              int32_t n_splits, tq_schedule schedule, float* out, float* lse_out,
                              float* part_o, float* part_lse, void* stream);

/* One decode step with its new token: the same result, bit for bit (cache and outputs), as
 * tq_quantize_append_kv(rot, keys, values, xk, xv, x_dtype, 1, pos, pos0, max_pos)
 * followed by tq_decode_attention over rows of length pos[b] + 1 (pos0 + 1 when pos is
 * NULL) with max_len = max_pos + 1 (pos0 + 1) and the remaining arguments as given
 * ("TurboQuant ...", 3.3: K and V are quantised on write and attention reads the
 * packed cache).  xk, xv: device [batch][n_kv_heads][1][128] of x_dtype; pos, pos0,
 * max_pos as for tq_quantize_append.  With the matrix-core schedule it is one launch: the
 * workgroups whose key-axis section holds a row's new position write that token before
 * reading the cache.  The vector schedule makes the two launches.  Errors: those of the
 * two calls it stands for; nothing is written when a check fails. */
tq_status tq_append_decode_attention(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                     const void* xk, const void* xv, tq_dtype x_dtype, const int32_t* pos,
                                     int32_t pos0, int32_t max_pos, const void* q, tq_dtype q_dtype,
                                     int32_t n_q_heads, float scale, int32_t n_splits, tq_schedule schedule,
                                     float* out, float* lse_out, float* part_o, float* part_lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the decode step of tq_append_decode_attention with
 * n_splits key-axis sections followed by tq_merge_splits, with the section partials held in a
 * library-owned static device buffer instead of caller buffers.  The result, cache bytes and
 * out/lse_out, equals that of tq_append_decode_attention(..., n_splits, part_o = P,
 * part_lse = L) followed by tq_merge_splits(rot, n_splits, keys->batch, n_q_heads, P, L, out,
 * lse_out) bit for bit; n_splits == 1 is tq_append_decode_attention itself.
 *   out: device [batch][n_q_heads][128] fp32; lse_out: device [batch][n_q_heads] or NULL.
 * The buffer holds TQ_STATIC_PARTIAL_FLOATS (1048576) floats per device, 4 MiB, allocated with
 * the library and kept until the process ends; its address is looked up once per device on
 * the first call there.  Nothing in it needs clearing: every section writes its partial.
 * Every call on a device shares that device's buffer, which keeps the last call's partials:
 * calls that overlap on one device (different streams, or host threads) race.  No memory is
 * allocated or freed by this call.
 * Errors: those of the two calls it stands for; TQ_ECAPACITY when n_splits * batch *
 * n_q_heads * 129 > TQ_STATIC_PARTIAL_FLOATS; TQ_EHIP when the buffer's address cannot be
 * obtained.  Nothing is written when a check fails. */
#define TQ_STATIC_PARTIAL_FLOATS (1 << 20)
tq_status tq_append_decode_attention_static(const tq_rotation* rot, const tq_cache* keys, const tq_cache* values,
                                            const void* xk, const void* xv, tq_dtype x_dtype, const int32_t* pos,
                                            int32_t pos0, int32_t max_pos, const void* q, tq_dtype q_dtype,
                                            int32_t n_q_heads, float scale, int32_t n_splits, tq_schedule schedule,
                                            float* out, float* lse_out, void* stream);

/* Attention over an unquantised K/V region, as key-axis section partials that merge with the
 * packed cache's: the prefill kept in fp16 while only decode-phase tokens are quantised
 * ("RotaryQuant ...", method overview, deferred prefill), or a window of recent tokens kept
 * unquantised ("RoPE-Aware Bit Allocation ...", results and limitations: the recent-token
 * buffer).  Softmax attention is a sum over tokens, so a row split between the two stores
 * is merged exactly by tq_merge_splits over all sections.
 *   k, v:     device [batch][n_kv_heads][capacity][128] of kv_dtype (TQ_F16 or TQ_F32);
 *             row b has seq_lens[b] tokens (device int32 [batch], each <= max_len) or max_len
 *             when seq_lens is NULL; max_len <= capacity.
 *   q:        device [batch][n_q_heads][128] of q_dtype; query head h reads KV head
 *             h / (n_q_heads / n_kv_heads).
 *   n_splits: sections as for tq_decode_attention: section s covers tokens [s*C,
 *             min(T, (s+1)*C)), C = ceil(T / n_splits).
 *   part_o, part_lse: written exactly as tq_decode_attention's partials
 *             ([n_splits][batch][n_q_heads][128] normalised and rotated forward by R, and
 *             [n_splits][batch][n_q_heads] natural-log lse; an empty section has lse = -inf
 *             and a zero partial).  Pointing them at section S of a larger partial buffer
 *             puts these sections after S packed ones for one tq_merge_splits call.
 * fp16 K/V run on the matrix cores: fp16 rows are exact operands against the query's fp16
 * high and low parts, weights enter the value product as fp16 high + low parts, with fp32
 * accumulation (scores and sums at fp32-level accuracy).  fp32 K/V are summed with fp32
 * fused multiply-adds.  Errors: TQ_EINVAL for null pointers, bad dtypes, counts or scale,
 * n_q_heads not a multiple of the rotation's KV heads; TQ_ECAPACITY for max_len > capacity
 * or capacity > TQ_MAX_CAPACITY. */
tq_status tq_dense_attention(const tq_rotation* rot, const void* k, const void* v, tq_dtype kv_dtype,
                             int32_t batch, int32_t capacity, const void* q, tq_dtype q_dtype,
                             int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                             int32_t n_splits, float* part_o, float* part_lse, void* stream);

/* Log-sum-exp merge of key-axis sections followed by the single inverse rotation:
 * lse = ln sum_s e^{lse_s}; out = R^T sum_s e^{lse_s - lse} part_o_s
 * ("RoPE-Aware Bit Allocation ...", packed-cache details; "RotaryQuant ...", key design 3).
 * part_o/part_lse as written by tq_decode_attention; out [batch][n_q_heads][128];
 * lse_out [batch][n_q_heads] or NULL.  n_q_heads must be a multiple of rot->n_kv_heads.
 * rot == NULL merges partials of the original domain (tq_zip_attention's) with no
 * rotation: out = sum_s e^{lse_s - lse} part_o_s. */
tq_status tq_merge_splits(const tq_rotation* rot, int32_t n_splits, int32_t batch, int32_t n_q_heads,
                          const float* part_o, const float* part_lse, float* out, float* lse_out,
                          void* stream);

/* ---- Lossless BF16 exponent codec of a KV cache ("ZipFusion: Fusing Lossless KV
 * Decompression with Attention ...", compression format, page metadata, register decode).
 *
 * A BF16 cache of [batch][n_kv_heads][tokens][128] (keys and values separately) is cut into
 * pages of 16 tokens; a page of one (sequence, KV head) is 4 chunks of 512 values, laid out
 * for the matrix products that read them (groups of 8 consecutive values are one thread's
 * operand): keys, chunk c = the page's tokens 4c .. 4c+3, token-major (a group = 8
 * coordinates of one token); values, chunk c = coordinates 32c .. 32c+31 of the page's 16
 * tokens, coordinate-major, value (d - 32c)*16 + t (a group = 8 tokens of one coordinate).
 * A chunk whose exponents all lie in [b, b+15], b = its smallest exponent rounded down to
 * even, is coded: its 512 low bytes (7 mantissa bits and the exponent's lowest bit) as they
 * are, then 256 code bytes, byte 4g+j holding value 8g+j (sign in bit 7, d = (exponent-b)/2
 * rounded down in bits 0-2) and value 8g+j+4 (sign bit 6, d bits 3-5): 768 bytes, 75% of
 * the original.  Any other chunk is kept as its 512 BF16 values (1024 bytes, same order).
 *   store: uint8 [batch][n_kv_heads][store_pages][4096]: page p's chunks back to back from
 *          the start of its 4096-byte slot; the slot's other bytes are zero.
 *   meta:  uint8 [batch][n_kv_heads][store_pages][8]: little-endian u32 byte offset of the
 *          page's first chunk within its (sequence, KV head) store (p * 4096 as written
 *          here), then one byte per chunk: 0xFF when kept, else b/2.
 * Decoding is exact: the high byte of a coded value is sign*128 + b/2 + d. */

/* Compresses n_pages whole pages of a BF16 token buffer of keys (role TQ_KEYS) or values
 * (TQ_VALUES) into a store.
 *   x:     device BF16 [batch][n_kv_heads][x_rows][128]; page i of the call is rows
 *          16*(src_page0+i) .. +15 and becomes store page dst_page0+i, for every
 *          (sequence, KV head).  A prefilled cache is compressed with x = the cache,
 *          src_page0 = dst_page0 = 0; a tail buffer of 16 rows that has just filled, with
 *          x_rows = 16, src_page0 = 0 and dst_page0 = its page number.
 *   store, meta: device, as above; only the n_pages pages are written.
 * Errors: TQ_EINVAL for null pointers, a bad role, non-positive counts or negative page
 * numbers; TQ_ECAPACITY when the pages pass x_rows or store_pages.  n_pages == 0 is a no-op. */
tq_status tq_zip_compress(const void* x, tq_role role, int32_t batch, int32_t n_kv_heads, int32_t x_rows, int32_t src_page0,
                          int32_t dst_page0, int32_t n_pages, uint8_t* store, uint8_t* meta, int32_t store_pages,
                          void* stream);

/* Decode attention read straight from the compressed pages: out = softmax(scale q K^T) V
 * over a row's T tokens, every stored value decoded in registers ("ZipFusion ...", fused
 * decompression and attention).  Pages 0 .. floor(T/16)-1 are read from the stores; the
 * T mod 16 tokens after them from the BF16 tail buffers, token t at row t mod tail_rows
 * (tail_rows = 16 for a buffer of the open page; a whole BF16 cache also serves, since
 * t mod tail_rows = t there).
 *   k_store, k_meta, v_store, v_meta: device, as written by tq_zip_compress; offsets read
 *          from the metadata are clamped so that a page slot stays inside the stream.
 *   k_tail, v_tail: device BF16 [batch][n_kv_heads][tail_rows][128], token-major for both
 *          roles; tail_rows a positive multiple of 16.
 *   q:     device [batch][n_q_heads][128] of q_dtype (TQ_F32, TQ_F16 or TQ_BF16); query
 *          head h reads KV head h / (n_q_heads / n_kv_heads); n_q_heads / n_kv_heads <= 8,
 *          or a multiple of 8.
 *   seq_lens: device int32 [batch] (each clamped to [0, max_len]) or NULL (all max_len);
 *          max_len <= 16 * store_pages + 15, and <= tail_rows when no page is stored.
 *   n_splits: key-axis sections of whole pages: section s covers tokens [s*C, min(T,
 *          (s+1)*C)), C = ceil(T / n_splits) rounded up to a multiple of 16.
 *   out, lse_out: n_splits == 1: device fp32 [batch][n_q_heads][128] and natural-log lse
 *          [batch][n_q_heads] (lse_out may be NULL); an empty row gives zeros and -inf.
 *   part_o, part_lse: n_splits > 1: fp32 [n_splits][batch][n_q_heads][128] normalised
 *          section outputs in the original domain and [n_splits][batch][n_q_heads] lse;
 *          tq_merge_splits with rot == NULL combines them.
 * Scores and sums are fp32.  Errors: TQ_EINVAL for null pointers, bad dtype, counts, scale
 * or head grouping; TQ_ECAPACITY when max_len passes the stored pages and the tail. */
tq_status tq_zip_attention(const uint8_t* k_store, const uint8_t* k_meta, const uint8_t* v_store,
                           const uint8_t* v_meta, int32_t store_pages, const void* k_tail, const void* v_tail,
                           int32_t tail_rows, int32_t batch, int32_t n_kv_heads, const void* q, tq_dtype q_dtype,
                           int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                           int32_t n_splits, float* out, float* lse_out, float* part_o, float* part_lse,
                           void* stream);

/* ---- Block-GTQ keys ("RoPE-Aware Bit Allocation for KV-Cache Quantization": overview,
 * block energy score, greedy allocation, grouping and packed-cache paragraphs).
 *
 * A head's 128 key coordinates form 64 RoPE blocks, block i = coordinates (2i, 2i+1).  Each
 * block gets an integer width b_i in [b_min, b_max] (1 <= b_min <= b_max <= 8, at most four
 * distinct widths per head: b_max - b_min <= 3 guarantees it) with
 * sum b_i = budget, greedily by the marginal gain (3/4) s_i 4^-b_i of the objective
 * sum s_i 4^-b_i, s_i the block's energy.  Blocks of equal width form one group, encoded by
 * one TQ-MSE encoder: the group's coordinates (its blocks' pairs in block order, n = 2 x
 * blocks) -> norm -> normalise -> y = Q^T u with a uniformly random rotation Q -> codes
 * by compare-count against the width's Lloyd-Max boundaries for n dimensions.  Values are
 * kept in fp16, the configuration of the page's main benchmark (keys only).
 *
 * Key record of one (token, KV head): code_bytes bytes of codes in group order (groups by
 * width ascending, each in its rotated coordinate order).  Groups of width <= 4 take nibble
 * containers, groups of width 5 .. 8 byte containers ("RoPE-Aware Bit Allocation ...",
 * packed-cache implementation details): the P positions of nibble groups first, position j
 * in byte j/2 (low nibble for even j), then one byte per position of the byte groups from
 * byte P/2, then zero padding.  code_bytes is one value for a whole cache: 64 when no head
 * has a group wider than 4 bits, else at least every head's tq_gtq_head.code_bytes (a
 * multiple of 16, at most 128).  Then norms[4] fp32, one per group (0 for absent groups). */
#define TQ_GTQ_BLOCKS 64
#define TQ_GTQ_MAX_GROUPS 4
#define TQ_GTQ_MAX_WIDTH 8
#define TQ_GTQ_ROTATION_FLOATS 16384 /* per head: every group's n x n rotation */

/* Block energies from a calibration prefix (host): energies[h][i] = 1/2 (mean over tokens
 * and the query heads reading KV head h of ||q^(i)||^2 + mean over tokens of ||k_h^(i)||^2),
 * block i = coordinates (2i, 2i+1), accumulated in double.
 *   q_cal: host float [n_tokens][n_q_heads][128]; k_cal: host float [n_tokens][n_kv_heads][128];
 *   energies: host float [n_kv_heads][64].
 * Errors: TQ_EINVAL for null pointers, non-positive counts or n_q_heads not a multiple of
 * n_kv_heads. */
tq_status tq_gtq_block_energies(const float* q_cal, const float* k_cal, int32_t n_tokens, int32_t n_q_heads,
                                int32_t n_kv_heads, float* energies);

/* Greedy integer allocation (host): bits[i] for n_blocks blocks with energies[i] >= 0.
 * Every block starts at b_min; each of the budget - n_blocks*b_min remaining bits goes to
 * the block below b_max with the largest (3/4) energies[i] 4^-bits[i] (in double; ties to
 * the lowest index).  Errors: TQ_EINVAL for null pointers, n_blocks <= 0, negative or
 * non-finite energies, b_min < 0, b_max < b_min, or a budget outside
 * [n_blocks*b_min, n_blocks*b_max]. */
tq_status tq_gtq_allocate(const float* energies, int32_t n_blocks, int32_t budget, int32_t b_min, int32_t b_max,
                          int32_t* bits);

/* One KV head's key encoder.  Plain data, copied to the device as an array per KV head. */
typedef struct {
  int32_t n_groups;                 /* 1 .. 4 */
  int32_t width[TQ_GTQ_MAX_GROUPS]; /* bits of group g, ascending */
  int32_t start[TQ_GTQ_MAX_GROUPS]; /* first group-order position of group g (128 if absent) */
  int32_t dim[TQ_GTQ_MAX_GROUPS];   /* coordinates of group g (0 if absent) */
  int32_t rot_offset[TQ_GTQ_MAX_GROUPS]; /* group g's rotation in the head's rotation array */
  int32_t coord[128];               /* original coordinate of group-order position j */
  int32_t byte_at[TQ_GTQ_MAX_GROUPS];  /* record byte of group g's first code */
  int32_t code_used;                /* code bytes the layout fills: P/2 + (128 - P) */
  int32_t code_bytes;               /* code_used rounded up to 16; 64 without byte groups */
  float centroid[TQ_GTQ_MAX_GROUPS][256];  /* 2^width levels each */
  float boundary[TQ_GTQ_MAX_GROUPS][255];
  float f16_scale[TQ_GTQ_MAX_GROUPS];  /* the codebook's tq_codebook.f16_scale: the matrix-core
                                          decode holds fp16(s c) and divides the query by s */
} tq_gtq_head;

/* Builds one head's encoder on the host from its 64 block widths (1 .. 8) and a Gaussian
 * matrix per width (gauss: float [max width][128][128], width w uses gauss[w-1]; only the
 * widths present are read).  Group g's rotation Q is the orthogonal factor, with positive
 * diagonal of R, of the leading n x n part of its width's matrix (QR by Gram-Schmidt in
 * double): a uniformly random rotation.  rotation: float [16384] (host), group g's Q
 * row-major at rot_offset[g] (Q[i][j] = rotation[rot_offset + i*n + j]; y_j = sum_i Q[i][j]
 * u_i).  Codebooks are tq_make_codebook(width, n) up to 4 bits; at 5 .. 8 bits the same
 * Lloyd-Max conditions ("TurboQuant ... MNN on phones", 2.3) solved by Newton's method.
 * Sets the record layout (byte_at, code_used, code_bytes; see the key record above).
 * Errors: TQ_EINVAL for null pointers or widths outside 1..8; TQ_EUNSUPPORTED for more than
 * four distinct widths. */
tq_status tq_gtq_prepare(const int32_t* block_bits, const float* gauss, tq_gtq_head* head, float* rotation);

/* Two-stage keys ("TurboQuant ... MNN on phones", 2.4 and 3.2: (b-1)-bit MSE plus a
 * 1-bit QJL residual whose sign bits give an unbiased inner-product estimate).  The first
 * stage is a Block-GTQ head whose 64 blocks all have width b - 1 (one group of the 128
 * coordinates in order, rotation Q); the second stores, per key, the m = 128 sign bits of
 * S r, r = x - x_hat the residual and S the m x 128 projection (independent N(0, 1)
 * entries, the caller's), and sqrt(pi/2)/m |r| in the record's norm slot 1.  The query's
 * score is <q, x_hat> + sqrt(pi/2)/m |r| sum_i (S q)_i sgn((S r)_i).
 * Since x = |x| Q y, r = |x| Q (y - c_hat) and S r = |x| (S Q)(y - c_hat); one matrix
 * M = S Q serves both the key encoding and the query (S q = M Q^T q).
 *
 * tq_gtq_qjl_projection (host): proj[j][i] = M[i][j] (M = S Q in double, stored fp32) for
 *   a head prepared by tq_gtq_prepare with every block at one width; S: [128][128]
 *   row-major; rotation: that head's rotation array.  TQ_EINVAL for another head layout. */
tq_status tq_gtq_qjl_projection(const tq_gtq_head* head, const float* rotation, const float* S, float* proj);

/* Encodes n_new keys per (sequence, KV head) into token positions pos0 .. pos0+n_new-1.
 *   heads:     device tq_gtq_head [n_kv_heads]; rotations: device float [n_kv_heads][16384].
 *   x:         device [batch][n_kv_heads][n_new][128] of x_dtype (TQ_F32 or TQ_F16).
 *   code_bytes: the record's code bytes (64, 80, 96, 112 or 128), the same for every head
 *              and at least each head's tq_gtq_head.code_bytes; a smaller value gives
 *              wrong codes for a head with byte groups but no access outside the record.
 *   codes:     device uint8 [batch][n_kv_heads][capacity][code_bytes] (padding written as
 *              zeros); norms: device float [batch][n_kv_heads][capacity][4].
 * Errors: TQ_EINVAL for null pointers, bad dtype, counts or code_bytes; TQ_ECAPACITY when
 * pos0 + n_new > capacity or capacity > TQ_MAX_CAPACITY.  n_new == 0 is a no-op. */
tq_status tq_gtq_quantize_keys(const tq_gtq_head* heads, const float* rotations, const void* x, tq_dtype x_dtype,
                               int32_t batch, int32_t n_kv_heads, int32_t n_new, int32_t pos0, int32_t capacity,
                               int32_t code_bytes, uint8_t* codes, float* norms, void* stream);

/* Decode attention over Block-GTQ keys and fp16 values: out = softmax(scale q K^T) V with
 * every key decoded from its codes, group norms and the rotated query (q~_g = Q_g^T q_g,
 * so q . k = sum_g norm_g sum_j q~_j c_g[code_j]).
 *   code_bytes, codes, norms: as tq_gtq_quantize_keys; v: device fp16
 *      [batch][n_kv_heads][capacity][128].
 *   q: device [batch][n_q_heads][128] of q_dtype (TQ_F32 or TQ_F16); n_q_heads a multiple
 *      of n_kv_heads, query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   seq_lens: device int32 [batch] (each clamped to [0, max_len]) or NULL (all max_len);
 *      max_len <= capacity.
 *   n_splits: key-axis sections as tq_decode_attention's: [s*C, min(T, (s+1)*C)),
 *      C = ceil(T / n_splits).
 *   out, lse_out: n_splits == 1: fp32 [batch][n_q_heads][128], natural-log lse (or NULL).
 *   part_o, part_lse: n_splits > 1: original-domain section partials for tq_merge_splits
 *      with rot == NULL.
 * Scores and weighted sums are fp16 matrix products of hi + lo parts (key levels, query,
 * weights) with fp32 accumulation; nibble codes are decoded two at a time through pair
 * tables, byte codes one at a time through a 256-entry table per group.  Errors: TQ_EINVAL
 * for null pointers, bad dtypes, counts, scale or code_bytes; TQ_ECAPACITY for max_len >
 * capacity or capacity > TQ_MAX_CAPACITY. */
tq_status tq_gtq_attention(const tq_gtq_head* heads, const float* rotations, int32_t code_bytes, const uint8_t* codes,
                           const float* norms,
                           const void* v, int32_t capacity, int32_t batch, int32_t n_kv_heads, const void* q,
                           tq_dtype q_dtype, int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                           int32_t n_splits, float* out, float* lse_out, float* part_o, float* part_lse, void* stream);

/* Two-stage keys (see tq_gtq_qjl_projection): the first stage's codes and norm as
 * tq_gtq_quantize_keys computes them with the one-group head, plus, per key, the 16 bytes of
 * sign bits of S r (bit i of the 128 in byte i/8 at bit i mod 8; a zero projection counts
 * as +) into signs [batch][n_kv_heads][capacity][16] and sqrt(pi/2)/128 |r| into norm slot 1.
 *   proj: device [n_kv_heads][128 * 128] from tq_gtq_qjl_projection.
 *   mse_bits: the first stage's width, which the heads were prepared with (1, 2 or 3; b - 1
 *      for b-bit keys, "TurboQuant ... MNN on phones", 3.2: the two stages take b bits per
 *      coordinate).  The codes are stored bit-packed at that width: codes
 *      [batch][n_kv_heads][capacity][16 * mse_bits], code of position i at bit offset
 *      mse_bits * i of the key's little-endian bit string (1 bit: byte i/8, bit i mod 8;
 *      2 bits: four codes per byte; 3 bits: eight codes in three bytes, sum_j c_j << 3j, the
 *      packed cache's unit).  A b-bit key thus takes 16 (b - 1) + 16 bytes of codes and
 *      signs plus two floats.  A value other than the heads' width gives wrong codes but no
 *      access outside the buffers (codes are capped at 2^mse_bits - 1).
 * Errors: those of tq_gtq_quantize_keys; TQ_EINVAL for a null proj or signs or mse_bits
 * outside 1..3. */
tq_status tq_gtq_qjl_quantize_keys(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                   int32_t mse_bits, const void* x,
                                   tq_dtype x_dtype, int32_t batch, int32_t n_kv_heads, int32_t n_new, int32_t pos0,
                                   int32_t capacity, uint8_t* codes, float* norms, uint8_t* signs, void* stream);

/* Decode attention over two-stage keys and fp16 values: as tq_gtq_attention, with each
 * score <q, x_hat> + sqrt(pi/2)/128 |r| sum_i (S q)_i sgn((S r)_i) (the projected query
 * S q = M Q^T q is formed once per workgroup; the signs are exact in fp16).  Arguments and
 * errors as tq_gtq_attention, plus proj, mse_bits (the codes' layout) and signs as
 * tq_gtq_qjl_quantize_keys (TQ_EINVAL when null or out of range).  With one-bit codes the
 * first stage's score is mid sum_j q~_j + half sum_j q~_j (+-1)_j for its two levels
 * mid -+ half, again with exact +-1 operands; 2- and 3-bit codes are decoded through one
 * table of the group's levels (four codes per entry at 2 bits, two at 3 bits). */
tq_status tq_gtq_qjl_attention(const tq_gtq_head* heads, const float* rotations, const float* proj,
                               int32_t mse_bits, const uint8_t* codes, const float* norms, const uint8_t* signs, const void* v,
                               int32_t capacity, int32_t batch, int32_t n_kv_heads, const void* q, tq_dtype q_dtype,
                               int32_t n_q_heads, const int32_t* seq_lens, int32_t max_len, float scale,
                               int32_t n_splits, float* out, float* lse_out, float* part_o, float* part_lse,
                               void* stream);

/* One decode step with its new token over Block-GTQ keys and fp16 values: the same cache
 * contents and outputs, bit for bit, as tq_gtq_quantize_keys of the new key at its slot and
 * a write of the new value row (converted to fp16 when x_dtype is TQ_F32), followed by
 * tq_gtq_attention over rows of length pos[b] + 1 (pos0 + 1 when pos is NULL) with max_len
 * = max_pos + 1 (pos0 + 1) ("RoPE-Aware Bit Allocation ...", packed-cache paragraph: keys
 * are encoded on write and the decode kernel reads the packed cache).  One launch: the
 * workgroups whose key-axis section holds a row's new slot write that token before reading
 * the cache.
 *   codes, norms, v: the cache, as tq_gtq_attention's, written at the new slots.
 *   k_new, v_new: device [batch][n_kv_heads][128] of x_dtype (TQ_F32 or TQ_F16).
 *   pos: device int32 [batch], each row's new slot, or NULL to use pos0 for every row;
 *      max_pos: host upper bound on pos[] (ignored when pos is NULL).  A device slot outside
 *      [0, max_pos] writes nothing and its row length is clamped as seq_lens' are.
 * Other arguments as tq_gtq_attention.  Errors: those of tq_gtq_attention; TQ_EINVAL for
 * null k_new or v_new, a bad x_dtype or a negative pos0 or max_pos; TQ_ECAPACITY when
 * max_pos + 1 (pos0 + 1) > capacity.  Nothing is written when a check fails. */
tq_status tq_gtq_append_attention(const tq_gtq_head* heads, const float* rotations, int32_t code_bytes, uint8_t* codes,
                                  float* norms,
                                  void* v, int32_t capacity, int32_t batch, int32_t n_kv_heads, const void* k_new,
                                  const void* v_new, tq_dtype x_dtype, const int32_t* pos, int32_t pos0,
                                  int32_t max_pos, const void* q, tq_dtype q_dtype, int32_t n_q_heads, float scale,
                                  int32_t n_splits, float* out, float* lse_out, float* part_o, float* part_lse,
                                  void* stream);

/* The decode step with its new token over two-stage keys: as tq_gtq_append_attention, with
 * the new key's sign bits and residual coefficient written too (tq_gtq_qjl_quantize_keys'
 * encoding, bit for bit) and attention as tq_gtq_qjl_attention.  Errors: those of
 * tq_gtq_append_attention; TQ_EINVAL for a null proj or signs or mse_bits outside 1..3. */
tq_status tq_gtq_qjl_append_attention(const tq_gtq_head* heads, const float* rotations, const float* proj,
                                      int32_t mse_bits, uint8_t* codes, float* norms, uint8_t* signs, void* v, int32_t capacity,
                                      int32_t batch, int32_t n_kv_heads, const void* k_new, const void* v_new,
                                      tq_dtype x_dtype, const int32_t* pos, int32_t pos0, int32_t max_pos,
                                      const void* q, tq_dtype q_dtype, int32_t n_q_heads, float scale,
                                      int32_t n_splits, float* out, float* lse_out, float* part_o, float* part_lse,
                                      void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H */

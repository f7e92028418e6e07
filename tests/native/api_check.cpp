// The C ABI's host code (tq_api.cpp with the codebook and Block-GTQ host code) over stub
// launchers: well-formed calls of every entry point reach exactly one launch with the
// arguments filled in; malformed, oversized and out-of-range ones are refused before any
// launch, with no undefined behaviour on the way (built with the address and
// undefined-behaviour sanitizers).  Device pointers are fake addresses: the host code never
// dereferences them.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "tq.h"
#include "tq_internal.h"

namespace tq {
extern int g_launches;
extern AppendArgs g_append;
extern DecodeArgs g_decode;
extern MergeArgs g_merge;
}  // namespace tq

#define CHECK(c)                                                          \
  do {                                                                    \
    if (!(c)) {                                                           \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(1);                                                       \
    }                                                                     \
  } while (0)

static void* const F = (void*)0x1000;  // a device address the host code must not touch
static float* const FF = (float*)0x1000;
static const int32_t* const FI = (const int32_t*)0x1000;

// call(expr) runs one entry point and returns (status, launches it made)
#define LAUNCHES(expr, st)             \
  ([&]() {                             \
    const int before = tq::g_launches; \
    st = (expr);                       \
    return tq::g_launches - before;    \
  })()

static tq_cache cache(tq_role role, int bits, int group, int batch, int heads, int capacity) {
  tq_cache c;
  c.codes = F;
  c.norms = FF;
  c.batch = batch;
  c.n_kv_heads = heads;
  c.capacity = capacity;
  c.bits = bits;
  c.group = group;
  c.role = role;
  CHECK(tq_make_codebook(bits, group, &c.codebook) == TQ_OK);
  return c;
}

static void packed() {
  tq_rotation rot{128, 8, FF, FF};
  tq_cache k = cache(TQ_KEYS, 3, 128, 4, 8, 4096), v = cache(TQ_VALUES, 3, 128, 4, 8, 4096);
  tq_status st;
  // well-formed: one launch each, arguments as given
  CHECK(LAUNCHES(tq_quantize_append(&rot, &k, F, TQ_F16, 100, nullptr, 7, 0, nullptr), st) == 1 && st == TQ_OK);
  CHECK(tq::g_append.pos0 == 7 && tq::g_append.n_new == 100 && tq::g_append.capacity == 4096);
  CHECK(LAUNCHES(tq_quantize_append_kv(&rot, &k, &v, F, F, TQ_F32, 4096, nullptr, 0, 0, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_decode_attention(&rot, &k, &v, F, TQ_F16, 32, FI, 4096, 0.1f, 8, TQ_SCHEDULE_AUTO, nullptr,
                                     nullptr, FF, FF, nullptr), st) == 1 && st == TQ_OK);
  CHECK(tq::g_decode.n_splits == 8 && tq::g_decode.group_size == 4 && tq::g_decode.n_slices == 1);
  CHECK(LAUNCHES(tq_append_decode_attention(&rot, &k, &v, F, F, TQ_F16, nullptr, 4095, 0, F, TQ_F32, 32, 0.1f, 1,
                                            TQ_SCHEDULE_VEC, FF, FF, nullptr, nullptr, nullptr), st) == 2 && st == TQ_OK);
  CHECK(LAUNCHES(tq_append_decode_attention(&rot, &k, &v, F, F, TQ_F16, nullptr, 4095, 0, F, TQ_F32, 32, 0.1f, 1,
                                            TQ_SCHEDULE_MFMA, FF, FF, nullptr, nullptr, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_merge_splits(&rot, 8, 4, 32, FF, FF, FF, FF, nullptr), st) == 1 && st == TQ_OK);
  CHECK(tq::g_merge.n_splits == 8);
  CHECK(LAUNCHES(tq_append_decode_attention_static(&rot, &k, &v, F, F, TQ_F16, nullptr, 100, 0, F, TQ_F16, 32, 0.1f,
                                                   8, TQ_SCHEDULE_AUTO, FF, nullptr, nullptr), st) == 2 && st == TQ_OK);
  CHECK(LAUNCHES(tq_dense_attention(&rot, F, F, TQ_F16, 4, 4096, F, TQ_F16, 32, nullptr, 4096, 0.1f, 8, FF, FF,
                                    nullptr), st) == 1 && st == TQ_OK);

  // malformed: refused, nothing launched
  tq_rotation bad_rot = rot;
  bad_rot.group = 64;
  CHECK(LAUNCHES(tq_quantize_append(&bad_rot, &k, F, TQ_F16, 1, nullptr, 0, 0, nullptr), st) == 0 && st != TQ_OK);
  CHECK(LAUNCHES(tq_quantize_append(&rot, &k, F, (tq_dtype)7, 1, nullptr, 0, 0, nullptr), st) == 0 && st == TQ_EINVAL);
  CHECK(LAUNCHES(tq_quantize_append(&rot, &k, F, TQ_F16, INT_MAX, nullptr, INT_MAX, 0, nullptr), st) == 0 &&
        st == TQ_ECAPACITY);
  CHECK(LAUNCHES(tq_quantize_append(&rot, &k, F, TQ_F16, 1, FI, 0, INT_MAX, nullptr), st) == 0 && st == TQ_ECAPACITY);
  CHECK(LAUNCHES(tq_decode_attention(&rot, &k, &v, F, TQ_F16, INT_MAX, nullptr, 10, 0.1f, INT_MAX,
                                     TQ_SCHEDULE_AUTO, FF, FF, FF, FF, nullptr), st) == 0 && st == TQ_EINVAL);
  CHECK(LAUNCHES(tq_decode_attention(&rot, &k, &v, F, TQ_F16, 32, nullptr, INT_MAX, 0.1f, 1,
                                     (tq_schedule)9, FF, FF, FF, FF, nullptr), st) == 0 && st != TQ_OK);
  CHECK(LAUNCHES(tq_append_decode_attention(&rot, &k, &v, F, F, TQ_F16, nullptr, INT_MAX, 0, F, TQ_F16, 32, 0.1f, 1,
                                            TQ_SCHEDULE_AUTO, FF, FF, nullptr, nullptr, nullptr), st) == 0 &&
        st == TQ_ECAPACITY);
  CHECK(LAUNCHES(tq_merge_splits(&rot, INT_MAX, INT_MAX, INT_MAX, FF, FF, FF, FF, nullptr), st) == 0 && st == TQ_EINVAL);
  CHECK(LAUNCHES(tq_dense_attention(&rot, F, F, TQ_F16, INT_MAX, INT_MAX, F, TQ_F16, 32, nullptr, 10, 0.1f, INT_MAX,
                                    FF, FF, nullptr), st) == 0 && st != TQ_OK);
  CHECK(LAUNCHES(tq_append_decode_attention_static(&rot, &k, &v, F, F, TQ_F16, nullptr, 100, 0, F, TQ_F16, 32, 0.1f,
                                                   INT_MAX, TQ_SCHEDULE_AUTO, FF, nullptr, nullptr), st) == 0 &&
        st != TQ_OK);
  tq_cache big = cache(TQ_KEYS, 4, 128, INT_MAX, 8, INT_MAX - 31);
  CHECK(LAUNCHES(tq_quantize_append(&rot, &big, F, TQ_F16, 1, nullptr, 0, 0, nullptr), st) == 0 && st != TQ_OK);
  big = cache(TQ_KEYS, 4, 128, 4, 8, TQ_MAX_CAPACITY + 32);
  CHECK(LAUNCHES(tq_quantize_append(&rot, &big, F, TQ_F16, 1, nullptr, 0, 0, nullptr), st) == 0 && st == TQ_ECAPACITY);
}

static void codecs() {
  tq_status st;
  uint8_t* const U = (uint8_t*)0x1000;
  CHECK(LAUNCHES(tq_zip_compress(F, TQ_KEYS, 2, 8, 8192, 0, 0, 512, U, U, 600, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_zip_compress(F, TQ_KEYS, 2, 8, INT_MAX, INT_MAX, INT_MAX, INT_MAX, U, U, INT_MAX, nullptr), st) == 0 &&
        st != TQ_OK);
  CHECK(LAUNCHES(tq_zip_attention(U, U, U, U, 512, F, F, 16, 2, 8, F, TQ_BF16, 32, nullptr, 8200, 0.1f, 1, FF, FF,
                                  nullptr, nullptr, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_zip_attention(U, U, U, U, INT_MAX, F, F, INT_MAX, 2, 8, F, TQ_BF16, 32, nullptr, INT_MAX, 0.1f,
                                  INT_MAX, FF, FF, FF, FF, nullptr), st) == 0 && st != TQ_OK);
  CHECK(LAUNCHES(tq_zip_attention(U, U, U, U, 512, F, F, 16, INT_MAX, INT_MAX, F, TQ_BF16, INT_MAX, nullptr, 8200,
                                  0.1f, INT_MAX, FF, FF, FF, FF, nullptr), st) == 0 && st == TQ_EINVAL);
  const tq_gtq_head* H = (const tq_gtq_head*)0x1000;
  CHECK(LAUNCHES(tq_gtq_quantize_keys(H, FF, F, TQ_F16, 4, 8, 100, 0, 32768, 64, U, FF, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_gtq_quantize_keys(H, FF, F, TQ_F16, 4, 8, INT_MAX, INT_MAX, INT_MAX, 64, U, FF, nullptr), st) == 0 &&
        st != TQ_OK);
  CHECK(LAUNCHES(tq_gtq_attention(H, FF, 80, U, FF, F, 32768, 4, 8, F, TQ_F16, 32, nullptr, 32768, 0.1f, 8, nullptr,
                                  nullptr, FF, FF, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_gtq_attention(H, FF, 80, U, FF, F, 32768, INT_MAX, 8, F, TQ_F16, INT_MAX - 7, nullptr, 32768,
                                  0.1f, INT_MAX, nullptr, nullptr, FF, FF, nullptr), st) == 0 && st != TQ_OK);
  CHECK(LAUNCHES(tq_gtq_append_attention(H, FF, 64, U, FF, F, 32768, 4, 8, F, F, TQ_F16, nullptr, 100, 0, F, TQ_F16,
                                         32, 0.1f, 3, nullptr, nullptr, FF, FF, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_gtq_qjl_quantize_keys(H, FF, FF, 2, F, TQ_F32, 4, 8, 100, 0, 32768, U, FF, U, nullptr), st) == 1 &&
        st == TQ_OK);
  CHECK(LAUNCHES(tq_gtq_qjl_quantize_keys(H, FF, FF, 4, F, TQ_F32, 4, 8, 100, 0, 32768, U, FF, U, nullptr), st) == 0 &&
        st == TQ_EINVAL);
  CHECK(LAUNCHES(tq_gtq_qjl_attention(H, FF, FF, 1, U, FF, U, F, 32768, 4, 8, F, TQ_F16, 32, nullptr, 32768, 0.1f, 1,
                                      FF, FF, nullptr, nullptr, nullptr), st) == 1 && st == TQ_OK);
  CHECK(LAUNCHES(tq_gtq_qjl_append_attention(H, FF, FF, 3, U, FF, U, F, 32768, 4, 8, F, F, TQ_F16, nullptr, 100, 0, F,
                                             TQ_F16, 32, 0.1f, 8, nullptr, nullptr, FF, FF, nullptr), st) == 1 &&
        st == TQ_OK);
}

int main() {
  packed();
  codecs();
  std::printf("api checks passed\n");
  return 0;
}

// Host-side entry points of the library built alone with address and undefined-behaviour
// sanitizers (the device launchers are not linked): codebooks, Block-GTQ allocation, encoder
// preparation, calibration energies and the two-stage projection, over valid and invalid
// arguments.  Exits non-zero on the first broken invariant; a sanitizer report aborts.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "tq.h"

#define CHECK(c)                                                    \
  do {                                                              \
    if (!(c)) {                                                     \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      std::exit(1);                                                 \
    }                                                               \
  } while (0)

static void codebooks() {
  const int dims[] = {2, 3, 8, 32, 128, 1024};
  for (int bits = 1; bits <= 8; ++bits)
    for (int dim : dims) {
      tq_codebook cb;
      const tq_status st = tq_make_codebook(bits, dim, &cb);
      if (bits > 4 && dim < 2) continue;
      if (st != TQ_OK) {
        // the packed cache's call takes 1..4 bits; wider codebooks come from tq_gtq_prepare
        CHECK(bits > 4 && st == TQ_EUNSUPPORTED);
        continue;
      }
      const int n = 1 << bits;
      for (int k = 0; k + 1 < n; ++k) {
        CHECK(cb.centroid[k] < cb.centroid[k + 1]);
        CHECK(std::fabs(cb.boundary[k] - 0.5f * (cb.centroid[k] + cb.centroid[k + 1])) <= 1e-6f);
      }
      CHECK(cb.f16_scale >= 1.f && cb.f16_scale < 2.f);
    }
  tq_codebook cb;
  CHECK(tq_make_codebook(0, 32, &cb) != TQ_OK);
  CHECK(tq_make_codebook(3, 1, &cb) != TQ_OK);
  CHECK(tq_make_codebook(3, 32, nullptr) == TQ_EINVAL);
  for (int s = 0; s <= 5; ++s) CHECK(tq_status_string((tq_status)s) != nullptr);
  CHECK(tq_status_string((tq_status)99) != nullptr);
}

static void allocation(std::mt19937& rng) {
  std::lognormal_distribution<float> ln(0.f, 2.f);
  for (int trial = 0; trial < 200; ++trial) {
    const int n = 1 + (int)(rng() % 64);
    const int b_min = (int)(rng() % 4), b_max = b_min + (int)(rng() % (9 - b_min));
    std::vector<float> e(n);
    for (auto& x : e) x = trial % 5 == 0 ? 1.f : ln(rng);  // ties in every fifth trial
    const int budget = n * b_min + (int)(rng() % (n * (b_max - b_min) + 1));
    std::vector<int32_t> bits(n, -1);
    CHECK(tq_gtq_allocate(e.data(), n, budget, b_min, b_max, bits.data()) == TQ_OK);
    int total = 0;
    for (int b : bits) {
      CHECK(b >= b_min && b <= b_max);
      total += b;
    }
    CHECK(total == budget);
  }
  std::vector<float> e(8, 1.f);
  std::vector<int32_t> bits(8);
  CHECK(tq_gtq_allocate(e.data(), 8, 8 * 9, 0, 8, bits.data()) != TQ_OK);  // above every block at b_max
  CHECK(tq_gtq_allocate(e.data(), 8, 7, 1, 4, bits.data()) != TQ_OK);      // below every block at b_min
  CHECK(tq_gtq_allocate(nullptr, 8, 16, 1, 4, bits.data()) == TQ_EINVAL);
  e[3] = -1.f;
  CHECK(tq_gtq_allocate(e.data(), 8, 16, 1, 4, bits.data()) != TQ_OK);     // negative energy
}

static void encoders(std::mt19937& rng) {
  std::normal_distribution<float> nd;
  std::vector<float> gauss((size_t)TQ_GTQ_MAX_WIDTH * 128 * 128);
  for (auto& x : gauss) x = nd(rng);
  std::vector<float> rot(TQ_GTQ_ROTATION_FLOATS), S(128 * 128), proj(128 * 128);
  for (auto& x : S) x = nd(rng);
  const int sets[][4] = {{1, 2, 3, 4}, {3, 5, 6, 0}, {2, 4, 7, 8}, {5, 0, 0, 0}, {8, 0, 0, 0}, {1, 0, 0, 0},
                         {4, 8, 0, 0}, {1, 8, 0, 0}};
  for (const auto& ws : sets) {
    int k = 0;
    while (k < 4 && ws[k]) ++k;
    std::vector<int32_t> bits(TQ_GTQ_BLOCKS);
    for (int i = 0; i < TQ_GTQ_BLOCKS; ++i) bits[i] = ws[(i * 7 + 3) % k];
    tq_gtq_head h;
    CHECK(tq_gtq_prepare(bits.data(), gauss.data(), &h, rot.data()) == TQ_OK);
    CHECK(h.n_groups == k);
    int dims = 0;
    for (int g = 0; g < h.n_groups; ++g) dims += h.dim[g];
    CHECK(dims == 128);
    CHECK(h.code_bytes >= 64 && h.code_bytes <= 128 && h.code_bytes % 16 == 0 && h.code_used <= h.code_bytes);
    for (float x : rot) CHECK(std::isfinite(x));
    const tq_status st = tq_gtq_qjl_projection(&h, rot.data(), S.data(), proj.data());
    CHECK(k == 1 ? st == TQ_OK : st == TQ_EINVAL);  // the two-stage keys' head is one group
  }
  std::vector<int32_t> five(TQ_GTQ_BLOCKS);
  for (int i = 0; i < TQ_GTQ_BLOCKS; ++i) five[i] = 1 + i % 5;
  tq_gtq_head h;
  CHECK(tq_gtq_prepare(five.data(), gauss.data(), &h, rot.data()) == TQ_EUNSUPPORTED);  // five widths
  five[0] = 9;
  CHECK(tq_gtq_prepare(five.data(), gauss.data(), &h, rot.data()) != TQ_OK);
}

static void energies(std::mt19937& rng) {
  std::normal_distribution<float> nd;
  const int n = 37, hq = 12, hkv = 3;
  std::vector<float> q((size_t)n * hq * 128), k((size_t)n * hkv * 128), e((size_t)hkv * TQ_GTQ_BLOCKS);
  for (auto& x : q) x = nd(rng);
  for (auto& x : k) x = nd(rng);
  CHECK(tq_gtq_block_energies(q.data(), k.data(), n, hq, hkv, e.data()) == TQ_OK);
  for (float x : e) CHECK(std::isfinite(x) && x >= 0.f);
  CHECK(tq_gtq_block_energies(q.data(), k.data(), n, 10, hkv, e.data()) != TQ_OK);  // 10 heads over 3
  CHECK(tq_gtq_block_energies(nullptr, k.data(), n, hq, hkv, e.data()) == TQ_EINVAL);
}

int main() {
  std::mt19937 rng(20260);
  codebooks();
  allocation(rng);
  encoders(rng);
  energies(rng);
  std::printf("host checks passed\n");
  return 0;
}

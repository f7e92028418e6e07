// Host-side Lloyd-Max codebook for the coordinate law of a uniformly rotated unit vector.
//
// "TurboQuant: ... MNN on phones", 2.2: after a uniform rotation one coordinate t of a
// point on the unit sphere in R^dim has density proportional to (1 - t^2)^((dim-3)/2)
// on [-1, 1].  2.3: the Lloyd-Max quantiser is one-dimensional continuous k-means on that
// law -- centroids are cell means, boundaries are midpoints of neighbouring centroids,
// iterated to convergence with the integrals done numerically.
//
// Cell masses use composite Gauss-Legendre quadrature (16 nodes per panel); the first
// moment has the closed form  int t (1-t^2)^mu dt = -(1-t^2)^(mu+1) / (2(mu+1)),  so a
// centroid is that difference over the mass.  The normalising constant cancels.  In two
// dimensions (mu = -1/2, the arcsine law, singular at the ends) the mass is also closed
// form: asin(hi) - asin(lo).
#include <cmath>
#include <cstring>

#include "tq.h"

namespace {

// 16-point Gauss-Legendre nodes/weights on [-1, 1] (positive half; symmetric).
const double kNodes[8] = {
    0.0950125098376374401853193, 0.2816035507792589132304605, 0.4580167776572273863424194,
    0.6178762444026437484466718, 0.7554044083550030338951012, 0.8656312023878317438804679,
    0.9445750230732325760779884, 0.9894009349916499325961542};
const double kWeights[8] = {
    0.1894506104550684962853967, 0.1826034150449235888667637, 0.1691565193950025381893121,
    0.1495959888165767320815017, 0.1246289712555338720524763, 0.0951585116824927848099251,
    0.0622535239386478928628438, 0.0271524594117540948517806};

double integrand(double t, double mu) {
  const double u = 1.0 - t * t;
  return u > 0.0 ? std::pow(u, mu) : 0.0;
}

// int_lo^hi (1 - t^2)^mu dt with `panels` equal Gauss-Legendre panels.
double mass(double lo, double hi, double mu, int panels) {
  if (hi <= lo) return 0.0;
  const double h = (hi - lo) / panels;
  double total = 0.0;
  for (int p = 0; p < panels; ++p) {
    const double a = lo + p * h, mid = a + 0.5 * h, half = 0.5 * h;
    double s = 0.0;
    for (int k = 0; k < 8; ++k) {
      s += kWeights[k] * (integrand(mid - half * kNodes[k], mu) + integrand(mid + half * kNodes[k], mu));
    }
    total += s * half;
  }
  return total;
}

double first_moment(double lo, double hi, double mu) {
  const double a = 1.0 - lo * lo, b = 1.0 - hi * hi;
  const double pa = a > 0 ? std::pow(a, mu + 1.0) : 0.0;
  const double pb = b > 0 ? std::pow(b, mu + 1.0) : 0.0;
  return (pa - pb) / (2.0 * (mu + 1.0));
}

}  // namespace

// The scale s in [1, 2) (a 2^-16 grid) at which every s * centroid lies closest, in the
// worst relative error over the levels, to an fp16 number.  Matrix-core decode stores the
// key codebook as fp16(s * c) and divides the query by s.
static float f16_scale(const float* centroid, int n) {
  float best = 1.f, best_err = INFINITY;
  for (int i = 0; i < 65536; ++i) {
    const float s = 1.f + (float)i / 65536.f;
    float err = 0.f;
    for (int k = 0; k < n; ++k) {
      const float v = s * centroid[k];
      if (v == 0.f) continue;
      const float r = (float)(_Float16)v;
      err = std::fmax(err, std::fabs(r - v) / std::fabs(v));
    }
    if (err < best_err) {
      best_err = err;
      best = s;
    }
  }
  return best;
}

extern "C" tq_status tq_make_codebook(int32_t bits, int32_t dim, tq_codebook* out) {
  if (out == nullptr) return TQ_EINVAL;
  if (bits < 1 || bits > 4 || dim < 2) return TQ_EUNSUPPORTED;
  const int n = 1 << bits;
  const double mu = 0.5 * (dim - 3);
  // the law has standard deviation 1/sqrt(dim): start from levels spread over +-2 sd, kept
  // inside (-1, 1) for the smallest dimensions
  double c[16], e[17];
  for (int k = 0; k < n; ++k)
    c[k] = dim < 4 ? -0.9 + 1.8 * k / (n - 1) : (-2.0 + 4.0 * k / (n - 1)) / std::sqrt((double)dim);
  for (int it = 0; it < 20000; ++it) {
    e[0] = -1.0;
    e[n] = 1.0;
    for (int k = 1; k < n; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
    double delta = 0.0;
    for (int k = 0; k < n; ++k) {
      const double m0 = dim == 2 ? std::asin(e[k + 1]) - std::asin(e[k]) : mass(e[k], e[k + 1], mu, 64);
      const double nc = m0 > 0.0 ? first_moment(e[k], e[k + 1], mu) / m0 : 0.5 * (e[k] + e[k + 1]);
      delta = std::fmax(delta, std::fabs(nc - c[k]));
      c[k] = nc;
    }
    if (delta < 1e-15) break;
  }
  // the law is even in t, so the quantiser is odd-symmetric: remove last-bit asymmetry so
  // that the middle boundary is exactly 0 (it decides the code of an exact zero)
  double sym[16];
  for (int k = 0; k < n; ++k) sym[k] = 0.5 * (c[k] - c[n - 1 - k]);
  for (int k = 0; k < n; ++k) c[k] = sym[k];
  std::memset(out, 0, sizeof(*out));
  out->bits = bits;
  out->dim = dim;
  for (int k = 0; k < n; ++k) out->centroid[k] = (float)c[k];
  for (int k = 0; k + 1 < n; ++k) out->boundary[k] = (float)(0.5 * (c[k] + c[k + 1]));
  out->f16_scale = f16_scale(out->centroid, n);
  return TQ_OK;
}

extern "C" const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_ECAPACITY: return "cache capacity exceeded";
    case TQ_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

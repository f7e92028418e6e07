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
#include <vector>

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

namespace tq {

// Lloyd-Max levels for 5 .. 8 bits (the byte containers of Block-GTQ keys): the conditions
// of 2.3 (each level the mean of its cell, boundaries at midpoints) solved by Newton's
// method, since the plain iteration above converges too slowly at 32 .. 256 levels.  The
// residual r_k = c_k - E[t | cell k] depends on c_{k-1}, c_k, c_{k+1} through the cell's two
// boundaries, so the Jacobian is tridiagonal (Thomas algorithm).  Cell integrals are taken
// in theta (t = sin theta): the mass of (1 - t^2)^mu dt is cos^(dim-2) theta d theta, smooth
// for every dim >= 2, by Gauss-Legendre panels; the first moment is closed form.  The start
// places levels at quantiles of the density^(1/3) law (the asymptotic point density of
// optimal quantisers, Panter and Dite).  Writes 2^bits centroids and 2^bits - 1 boundaries
// (fp32) and the fp16 scale; returns false if the iteration does not settle.
bool wide_codebook(int bits, int dim, float* centroid, float* boundary, float* scale) {
  if (bits < 5 || bits > 8 || dim < 2) return false;
  const int n = 1 << bits;
  const double mu = 0.5 * (dim - 3), pw = dim - 2.0;
  auto cos_mass = [&](double lo, double hi) {  // int_lo^hi (1 - t^2)^mu dt
    const double a = std::asin(std::fmax(-1.0, std::fmin(1.0, lo))), b = std::asin(std::fmax(-1.0, std::fmin(1.0, hi)));
    if (b <= a) return 0.0;
    const int panels = 8;
    const double h = (b - a) / panels;
    double total = 0.0;
    for (int p = 0; p < panels; ++p) {
      const double mid = a + (p + 0.5) * h, half = 0.5 * h;
      double sum = 0.0;
      for (int k = 0; k < 8; ++k)
        sum += kWeights[k] * (std::pow(std::cos(mid - half * kNodes[k]), pw) + std::pow(std::cos(mid + half * kNodes[k]), pw));
      total += sum * half;
    }
    return total;
  };
  auto dens = [&](double t) { return integrand(t, mu); };
  // start: quantiles of f^(1/3), integrated in theta (f^(1/3) dt = cos^(dim/3) theta d theta)
  const int G = 20000;
  std::vector<double> cum(G + 1);
  cum[0] = 0.0;
  for (int i = 0; i < G; ++i) {
    const double t0 = -M_PI / 2 + M_PI * i / G, t1 = -M_PI / 2 + M_PI * (i + 1) / G;
    cum[i + 1] = cum[i] + 0.5 * (std::pow(std::cos(t0), dim / 3.0) + std::pow(std::cos(t1), dim / 3.0)) * (t1 - t0);
  }
  double c[256], m0[256], mean[256], b[256], res[256];
  for (int k = 0, i = 0; k < n; ++k) {
    const double target = (k + 0.5) / n * cum[G];
    while (i < G - 1 && cum[i + 1] < target) ++i;
    const double f = (target - cum[i]) / (cum[i + 1] - cum[i]);
    c[k] = std::sin(-M_PI / 2 + M_PI * (i + f) / G);
  }
  for (int it = 0; it < 100; ++it) {
    for (int k = 0; k + 1 < n; ++k) b[k] = 0.5 * (c[k] + c[k + 1]);
    double worst = 0.0;
    for (int k = 0; k < n; ++k) {
      const double lo = k ? b[k - 1] : -1.0, hi = k + 1 < n ? b[k] : 1.0;
      m0[k] = cos_mass(lo, hi);
      mean[k] = first_moment(lo, hi, mu) / m0[k];
      res[k] = c[k] - mean[k];
      worst = std::fmax(worst, std::fabs(res[k]));
    }
    if (worst < 1e-13) break;
    // tridiagonal Jacobian: d mean_k / d b = (b - mean_k) f(b) / m0_k at the upper boundary,
    // minus that at the lower one; a boundary moves by half of either neighbouring level
    double lo_d[256], di[256], up_d[256];
    for (int k = 0; k < n; ++k) {
      di[k] = 1.0;
      lo_d[k] = up_d[k] = 0.0;
      if (k + 1 < n) {
        const double u = (b[k] - mean[k]) * dens(b[k]) / (2.0 * m0[k]);
        di[k] -= u;
        up_d[k] = -u;
      }
      if (k > 0) {
        const double l = (b[k - 1] - mean[k]) * dens(b[k - 1]) / (2.0 * m0[k]);
        di[k] += l;
        lo_d[k] = l;
      }
    }
    // Thomas algorithm
    double cp[256], dp[256], step[256];
    cp[0] = up_d[0] / di[0];
    dp[0] = res[0] / di[0];
    for (int k = 1; k < n; ++k) {
      const double den = di[k] - lo_d[k] * cp[k - 1];
      cp[k] = up_d[k] / den;
      dp[k] = (res[k] - lo_d[k] * dp[k - 1]) / den;
    }
    step[n - 1] = dp[n - 1];
    for (int k = n - 2; k >= 0; --k) step[k] = dp[k] - cp[k] * step[k + 1];
    double lam = 1.0, nc[256];
    for (int tries = 0; tries < 60; ++tries, lam *= 0.5) {
      bool ok = true;
      for (int k = 0; k < n; ++k) nc[k] = c[k] - lam * step[k];
      for (int k = 0; k < n && ok; ++k) ok = nc[k] > -1.0 && nc[k] < 1.0 && (k == 0 || nc[k] > nc[k - 1]);
      if (ok) break;
    }
    for (int k = 0; k < n; ++k) c[k] = nc[k];
  }
  double worst = 0.0;
  for (int k = 0; k < n; ++k) worst = std::fmax(worst, std::fabs(res[k]));
  if (!(worst < 1e-10)) return false;
  double sym[256];
  for (int k = 0; k < n; ++k) sym[k] = 0.5 * (c[k] - c[n - 1 - k]);
  for (int k = 0; k < n; ++k) centroid[k] = (float)sym[k];
  for (int k = 0; k + 1 < n; ++k) boundary[k] = (float)(0.5 * (sym[k] + sym[k + 1]));
  *scale = f16_scale(centroid, n);
  return true;
}

}  // namespace tq

extern "C" const char* tq_status_string(tq_status s) {
  switch (s) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_EUNSUPPORTED: return "unsupported configuration";
    case TQ_ECAPACITY: return "cache capacity exceeded";
    case TQ_EHIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

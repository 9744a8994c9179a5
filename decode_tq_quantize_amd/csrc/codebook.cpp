// Lloyd-Max codebook on the rotated-coordinate marginal (host, fp64).
//
// riverfrot "TurboQuant" post, section 4.1: after the random rotation every
// coordinate of the unit vector follows one Beta-type law; section 4.2:
// Lloyd-Max takes that density and 2^b levels and returns boundaries {t_i}
// and representatives {c_i}, computed once per (d, b).
//
// The law used is the exact marginal of a coordinate of a uniform point on
// the unit sphere in R^d: f_d(x) = C_d (1 - x^2)^((d-3)/2), i.e.
// (x + 1) / 2 ~ Beta(a, a) with a = (d - 1) / 2. The density is even and
// log-concave, so the Lloyd-Max fixed point is unique and symmetric: this
// implementation iterates on the non-negative half only (0 is a boundary
// when L is even) and mirrors the result.
#include <cmath>
#include <vector>

#include "tq.h"

namespace tq_host {

// Continued fraction of the regularised incomplete beta function
// (the even/odd coefficient expansion, evaluated by the modified Lentz
// method). Converges fast for x < (a + 1) / (a + b + 2).
static double beta_cf(double a, double b, double x) {
  const double tiny = 1e-300;
  const double eps = 1e-16;
  double f = 1.0, C = 1.0, D = 0.0;
  for (int j = 1; j < 100000; ++j) {
    double coef;
    if (j & 1) {
      const double m = (j - 1) / 2;
      coef = -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
    } else {
      const double m = j / 2;
      coef = m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    }
    D = 1.0 + coef * D;
    if (std::fabs(D) < tiny) D = tiny;
    C = 1.0 + coef / C;
    if (std::fabs(C) < tiny) C = tiny;
    D = 1.0 / D;
    const double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < eps) break;
  }
  return 1.0 / f;
}

// I_x(a, b), regularised.
static double inc_beta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lbeta = std::lgamma(a) + std::lgamma(b) - std::lgamma(a + b);
  if (x < (a + 1.0) / (a + b + 2.0)) {
    const double pre = std::exp(a * std::log(x) + b * std::log1p(-x) - lbeta);
    return pre * beta_cf(a, b, x) / a;
  }
  const double pre = std::exp(b * std::log1p(-x) + a * std::log(x) - lbeta);
  return 1.0 - pre * beta_cf(b, a, 1.0 - x) / b;
}

// Upper tail P(X >= x) for x >= 0.
static double upper_tail(int d, double x) {
  const double a = 0.5 * (d - 1);
  return inc_beta(a, a, 0.5 * (1.0 - x));
}

// log C_d, C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)).
static double log_norm(int d) {
  return std::lgamma(0.5 * d) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (d - 1));
}

// Integral of x f_d(x) over [lo, hi] (0 <= lo < hi <= 1):
// C_d [(1 - lo^2)^((d-1)/2) - (1 - hi^2)^((d-1)/2)] / (d - 1).
static double first_moment(int d, double lo, double hi) {
  const double e = 0.5 * (d - 1);
  auto g = [&](double x) { return x >= 1.0 ? 0.0 : std::exp(e * std::log1p(-x * x)); };
  return std::exp(log_norm(d)) * (g(lo) - g(hi)) / (d - 1);
}

}  // namespace tq_host

extern "C" int tq_build_codebook(int d, int mse_bits, double* centroids, double* thresholds,
                                 double* mse_out, int max_iter) {
  using namespace tq_host;
  if (!centroids || !thresholds) return TQ_ERR_INVALID_ARG;
  if (d < 3 || d > TQ_MAX_DIM || mse_bits < 1 || mse_bits > TQ_MAX_MSE_BITS) return TQ_ERR_UNSUPPORTED;
  if (max_iter < 0) return TQ_ERR_INVALID_ARG;
  if (max_iter == 0) max_iter = 200000;
  const int L = 1 << mse_bits;
  const int H = L / 2;  // levels on the positive side
  // positive centroids c[0] < ... < c[H-1]; boundaries 0 = b[0] < b[1..H-1] < b[H] = 1
  std::vector<double> c(H), b(H + 1);
  const double span = std::fmin(2.0 / std::sqrt((double)d), 1.0 - 1.0 / L);
  for (int i = 0; i < H; ++i) c[i] = span * (2.0 * i + 1.0) / (2.0 * H - 1.0) * (H > 1 ? 1.0 : 0.5);
  bool converged = false;
  for (int it = 0; it < max_iter; ++it) {
    b[0] = 0.0;
    b[H] = 1.0;
    for (int i = 1; i < H; ++i) b[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0;
    for (int i = 0; i < H; ++i) {
      const double mass = upper_tail(d, b[i]) - upper_tail(d, b[i + 1]);
      const double cn = first_moment(d, b[i], b[i + 1]) / mass;
      if (!std::isfinite(cn)) return TQ_ERR_NO_CONVERGE;
      delta = std::fmax(delta, std::fabs(cn - c[i]));
      c[i] = cn;
    }
    if (delta < 1e-14) {
      converged = true;
      break;
    }
  }
  if (!converged) return TQ_ERR_NO_CONVERGE;
  for (int i = 0; i < H; ++i) {
    centroids[H + i] = c[i];
    centroids[H - 1 - i] = -c[i];
  }
  for (int i = 0; i < L - 1; ++i) thresholds[i] = 0.5 * (centroids[i] + centroids[i + 1]);
  thresholds[H - 1] = 0.0;
  if (mse_out) {
    // At the centroid condition E[(X - Q(X))^2] = E[X^2] - sum_k c_k^2 P_k,
    // with E[X^2] = 1/d; D is d times that (error of a unit vector).
    double s = 0.0;
    for (int i = 0; i < H; ++i) {
      const double lo = i == 0 ? 0.0 : 0.5 * (c[i - 1] + c[i]);
      const double hi = i == H - 1 ? 1.0 : 0.5 * (c[i] + c[i + 1]);
      s += 2.0 * c[i] * c[i] * (upper_tail(d, lo) - upper_tail(d, hi));
    }
    *mse_out = 1.0 - d * s;
  }
  return TQ_OK;
}

extern "C" int tq_quantizer_init(tq_quantizer* q, int d, int mse_bits, tq_variant variant,
                                 const float* R, const float* S) {
  if (!q) return TQ_ERR_INVALID_ARG;
  if (d < 32 || d > TQ_MAX_DIM || (d % 32) != 0) return TQ_ERR_UNSUPPORTED;
  if (variant != TQ_MSE && variant != TQ_PROD) return TQ_ERR_INVALID_ARG;
  double c[TQ_MAX_LEVELS], t[TQ_MAX_LEVELS - 1];
  const int rc = tq_build_codebook(d, mse_bits, c, t, nullptr, 0);
  if (rc != TQ_OK) return rc;
  tq_quantizer out{};
  out.d = d;
  out.mse_bits = mse_bits;
  out.variant = variant;
  out.R = R;
  out.S = variant == TQ_PROD ? S : nullptr;
  const int L = 1 << mse_bits;
  for (int i = 0; i < L; ++i) out.centroids[i] = (float)c[i];
  for (int i = 0; i < L - 1; ++i) out.thresholds[i] = (float)t[i];
  *q = out;
  return TQ_OK;
}

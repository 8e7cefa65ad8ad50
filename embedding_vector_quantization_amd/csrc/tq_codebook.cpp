// Host-side Lloyd-Max codebook for the Lemma 1 density.
//
// Source: "TurboQuant: Online Vector Quantization" paper summary (Jump2Paper
// Archive) -- Lemma 1 gives the marginal of one coordinate of a uniform point
// on S^{d-1}:
//     f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - x^2)^((d-3)/2);
// the MSE decomposition reduces D_mse to d * C(f_X, b), the optimal 1-D
// k-means cost of f_X with 2^b levels; the experiment-setup table says the
// codebooks are precomputed by numerical Max-Lloyd optimisation.
//
// f_X is even and log-concave (d >= 3), so the optimum is unique and
// odd-symmetric.  We work on the positive half: H = 2^(m-1) centroids
// 0 < c_0 < ... < c_{H-1}, cell edges e_0 = 0, e_k = (c_{k-1} + c_k)/2,
// e_H = 1.  The Lloyd map is L_k(c) = int_cell x f / int_cell f.  The fixed
// point is reached by a few Lloyd steps from a companding start and then by
// damped Newton steps on c - L(c) = 0, whose Jacobian is tridiagonal:
//     dL_k/de_{k+1} =  f(e_{k+1}) (e_{k+1} - L_k) / M0_k
//     dL_k/de_k     = -f(e_k)     (e_k     - L_k) / M0_k
// with de_k/dc_{k-1} = de_k/dc_k = 1/2.  Integrals use composite
// Gauss-Legendre quadrature on panels a fraction of 1/sqrt(d) wide.

#include <algorithm>
#include <cmath>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr int kGaussNodes = 20;

struct GaussLegendre {
  double x[kGaussNodes];
  double w[kGaussNodes];
  GaussLegendre() {
    // Roots of P_n by Newton's method from the Chebyshev-like start
    // cos(pi (i + 3/4) / (n + 1/2)); weights 2 / ((1 - x^2) P_n'(x)^2).
    const int n = kGaussNodes;
    for (int i = 0; i < n; ++i) {
      double z = std::cos(M_PI * (i + 0.75) / (n + 0.5));
      double dp = 0.0;
      for (int it = 0; it < 100; ++it) {
        double p0 = 1.0, p1 = z;
        for (int k = 2; k <= n; ++k) {
          double pk = ((2.0 * k - 1.0) * z * p1 - (k - 1.0) * p0) / k;
          p0 = p1;
          p1 = pk;
        }
        dp = n * (z * p1 - p0) / (z * z - 1.0);
        double dz = p1 / dp;
        z -= dz;
        if (std::fabs(dz) < 1e-16) break;
      }
      x[i] = z;
      w[i] = 2.0 / ((1.0 - z * z) * dp * dp);
    }
  }
};

const GaussLegendre &gauss() {
  static const GaussLegendre g;
  return g;
}

class BetaMarginal {
 public:
  explicit BetaMarginal(int d)
      : d_(d),
        expo_(0.5 * (d - 3)),
        log_norm_(std::lgamma(0.5 * d) - 0.5 * std::log(M_PI) - std::lgamma(0.5 * (d - 1))),
        panel_(0.25 / std::sqrt(static_cast<double>(d))) {}

  double pdf(double x) const {
    if (x <= -1.0 || x >= 1.0) return 0.0;
    if (expo_ == 0.0) return std::exp(log_norm_);
    return std::exp(log_norm_ + expo_ * std::log1p(-x * x));
  }

  // Integrals over [a, b] (0 <= a < b <= 1) of f, x f and (x - c)^2 f.
  void moments(double a, double b, double c, double *m0, double *m1, double *m2) const {
    const GaussLegendre &g = gauss();
    double s0 = 0.0, s1 = 0.0, s2 = 0.0;
    // Beyond ~40 standard deviations the density is below 1e-300.
    const double cutoff = std::min(1.0, 40.0 / std::sqrt(static_cast<double>(d_)) + 1e-3);
    double hi = std::min(b, std::max(cutoff, a));
    if (d_ <= 8) hi = b;
    int panels = static_cast<int>(std::ceil((hi - a) / panel_));
    panels = std::max(1, std::min(panels, 4096));
    const double h = (hi - a) / panels;
    for (int p = 0; p < panels; ++p) {
      const double lo = a + p * h;
      const double mid = lo + 0.5 * h;
      for (int i = 0; i < kGaussNodes; ++i) {
        const double x = mid + 0.5 * h * g.x[i];
        const double fw = pdf(x) * g.w[i] * 0.5 * h;
        s0 += fw;
        s1 += x * fw;
        s2 += (x - c) * (x - c) * fw;
      }
    }
    *m0 = s0;
    *m1 = s1;
    *m2 = s2;
  }

 private:
  int d_;
  double expo_;
  double log_norm_;
  double panel_;
};

double normal_quantile(double p) {
  // Bisection on the standard normal CDF 0.5 * erfc(-x / sqrt 2).
  double lo = -40.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct LloydState {
  std::vector<double> edges, m0, lmap, fe;  // fe[k] = f(e_k)
};

void lloyd_eval(const BetaMarginal &f, const std::vector<double> &c, LloydState *st) {
  const int h = static_cast<int>(c.size());
  st->edges.assign(h + 1, 0.0);
  st->edges[0] = 0.0;
  for (int k = 1; k < h; ++k) st->edges[k] = 0.5 * (c[k - 1] + c[k]);
  st->edges[h] = 1.0;
  st->m0.assign(h, 0.0);
  st->lmap.assign(h, 0.0);
  st->fe.assign(h + 1, 0.0);
  for (int k = 0; k < h; ++k) {
    double a0, a1, a2;
    f.moments(st->edges[k], st->edges[k + 1], 0.0, &a0, &a1, &a2);
    st->m0[k] = a0;
    st->lmap[k] = a0 > 0.0 ? a1 / a0 : 0.5 * (st->edges[k] + st->edges[k + 1]);
  }
  for (int k = 0; k <= h; ++k) st->fe[k] = f.pdf(st->edges[k]);
}

bool increasing_positive(const std::vector<double> &c) {
  if (c.empty() || !(c[0] > 0.0)) return false;
  for (size_t k = 1; k < c.size(); ++k)
    if (!(c[k] > c[k - 1])) return false;
  return c.back() < 1.0;
}

}  // namespace

int make_codebook(int d, int m, double *centroids, double *thresholds, double *dmse) {
  const int h = 1 << (m - 1);
  const BetaMarginal f(d);
  // Companding start: the high-resolution point density is proportional to
  // f^(1/3); for the near-Gaussian f_X that is N(0, 3/d).
  std::vector<double> c(h);
  const double s3 = std::sqrt(3.0 / d);
  for (int k = 0; k < h; ++k) {
    const double p = 0.5 + 0.5 * (k + 0.5) / h;
    c[k] = std::min(0.99, s3 * normal_quantile(p));
  }
  LloydState st;
  for (int it = 0; it < 60; ++it) {
    lloyd_eval(f, c, &st);
    c = st.lmap;
  }
  // Damped Newton on F(c) = c - L(c).
  double resid = 1.0;
  for (int it = 0; it < 200; ++it) {
    lloyd_eval(f, c, &st);
    std::vector<double> rhs(h), lower(h, 0.0), diag(h, 1.0), upper(h, 0.0);
    resid = 0.0;
    for (int k = 0; k < h; ++k) {
      rhs[k] = st.lmap[k] - c[k];
      resid = std::max(resid, std::fabs(rhs[k]));
    }
    if (resid < 1e-16) break;
    for (int k = 0; k < h; ++k) {
      const double mk = st.m0[k];
      if (!(mk > 0.0)) continue;
      const double d_hi = st.fe[k + 1] * (st.edges[k + 1] - st.lmap[k]) / mk;  // dL_k/de_{k+1}
      const double d_lo = -st.fe[k] * (st.edges[k] - st.lmap[k]) / mk;        // dL_k/de_k
      // J = dL/dc; the system is (I - J) delta = L - c.
      if (k >= 1) {
        lower[k] -= 0.5 * d_lo;
        diag[k] -= 0.5 * d_lo;
      }
      if (k + 1 <= h - 1) {
        diag[k] -= 0.5 * d_hi;
        upper[k] -= 0.5 * d_hi;
      }
    }
    // Thomas algorithm.
    std::vector<double> cp(h), dp(h), delta(h);
    cp[0] = upper[0] / diag[0];
    dp[0] = rhs[0] / diag[0];
    for (int k = 1; k < h; ++k) {
      const double den = diag[k] - lower[k] * cp[k - 1];
      cp[k] = upper[k] / den;
      dp[k] = (rhs[k] - lower[k] * dp[k - 1]) / den;
    }
    delta[h - 1] = dp[h - 1];
    for (int k = h - 2; k >= 0; --k) delta[k] = dp[k] - cp[k] * delta[k + 1];
    double step = 1.0;
    std::vector<double> trial(h);
    bool accepted = false;
    for (int halving = 0; halving < 40; ++halving) {
      for (int k = 0; k < h; ++k) trial[k] = c[k] + step * delta[k];
      if (increasing_positive(trial)) {
        LloydState ts;
        lloyd_eval(f, trial, &ts);
        double r2 = 0.0;
        for (int k = 0; k < h; ++k) r2 = std::max(r2, std::fabs(ts.lmap[k] - trial[k]));
        if (r2 < resid || r2 < 1e-16) {
          accepted = true;
          break;
        }
      }
      step *= 0.5;
    }
    if (!accepted) {
      c = st.lmap;  // fall back to a plain Lloyd step
    } else {
      c = trial;
    }
  }
  lloyd_eval(f, c, &st);
  resid = 0.0;
  for (int k = 0; k < h; ++k) resid = std::max(resid, std::fabs(st.lmap[k] - c[k]));
  if (!(resid < 1e-13) || !increasing_positive(c)) return TQ_ERR_NOCONV;

  double cost = 0.0;
  for (int k = 0; k < h; ++k) {
    double a0, a1, a2;
    f.moments(st.edges[k], st.edges[k + 1], c[k], &a0, &a1, &a2);
    cost += a2;
  }
  const int K = 2 * h;
  for (int k = 0; k < h; ++k) {
    centroids[h + k] = c[k];
    centroids[h - 1 - k] = -c[k];
  }
  thresholds[h - 1] = 0.0;
  for (int k = 1; k < h; ++k) {
    thresholds[h - 1 + k] = st.edges[k];
    thresholds[h - 1 - k] = -st.edges[k];
  }
  (void)K;
  if (dmse) *dmse = 2.0 * d * cost;
  return TQ_OK;
}

}  // namespace tq

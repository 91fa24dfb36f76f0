// Host Lloyd-Max codebook builder for the TurboQuant MSE codec.
//
// "TurboQuant KV Cache Quantization in MLX-VLM", section "How TurboQuant KV
// Cache Quantization Works": the codec's codebook is a Lloyd-Max quantizer
// fitted to a Beta-shaped density.  The density used is the exact marginal
// of one coordinate of a uniformly random unit vector in R^d,
//   f_d(x) = C_d (1 - x^2)^((d - 3)/2),  C_d = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)),
// i.e. (1 + X)/2 ~ Beta((d-1)/2, (d-1)/2); a rotated unit vector has exactly
// this marginal in every coordinate.
//
// Lloyd-Max: thresholds at the midpoints of neighbouring centroids, each
// centroid the conditional mean of its cell; iterate to the fixed point
// (unique, since f_d is log-concave).  The density is even, so only the
// positive half is iterated and the codebook is mirrored; the middle
// threshold is then exactly 0.
//
// Cell probabilities use the regularized incomplete beta function evaluated
// by its continued fraction (DLMF 8.17.22) with the modified Lentz algorithm
// (Lentz 1976; Thompson and Barnett 1986).  Cell first moments have the
// closed form F1(lo) - F1(hi) with F1(x) = C_d (1 - x^2)^((d-1)/2) / (d - 1).
#include <cmath>
#include <cstdint>
#include <vector>

#include "tq.h"

namespace {

// Continued fraction of DLMF 8.17.22 for the regularized incomplete beta:
//   I_x(a, b) = x^a (1 - x)^b / (a B(a, b)) / g,
//   g = 1 + d_1/(1 + d_2/(1 + ...)),
//   d_{2m+1} = -(a + m)(a + b + m) x / ((a + 2m)(a + 2m + 1)),
//   d_{2m}   =  m (b - m) x / ((a + 2m - 1)(a + 2m)).
// g is evaluated forwards with the modified Lentz algorithm.  The fraction
// converges quickly for x < (a + 1)/(a + b + 2).
double incbeta_fraction(double a, double b, double x) {
  const double tiny = 1e-300;
  const double eps = 1e-15;
  double g = 1.0, C = 1.0, D = 0.0;
  for (int j = 1; j < 1000000; ++j) {
    const int m = j / 2;
    double dj;
    if (j & 1) {
      dj = -((a + m) * (a + b + m) * x) / ((a + 2.0 * m) * (a + 2.0 * m + 1.0));
    } else {
      dj = (m * (b - m) * x) / ((a + 2.0 * m - 1.0) * (a + 2.0 * m));
    }
    D = 1.0 + dj * D;
    if (std::fabs(D) < tiny) D = tiny;
    C = 1.0 + dj / C;
    if (std::fabs(C) < tiny) C = tiny;
    D = 1.0 / D;
    const double delta = C * D;
    g *= delta;
    if (std::fabs(delta - 1.0) < eps) break;
  }
  return g;
}

// Regularized incomplete beta I_x(a, b), using I_x(a, b) = 1 - I_{1-x}(b, a)
// on the side where the fraction converges slowly.
double incbeta(double a, double b, double x) {
  if (x <= 0.0) return 0.0;
  if (x >= 1.0) return 1.0;
  const double lfront = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) +
                        a * std::log(x) + b * std::log1p(-x);
  if (x < (a + 1.0) / (a + b + 2.0)) {
    return std::exp(lfront) / a / incbeta_fraction(a, b, x);
  }
  const double lback = std::lgamma(a + b) - std::lgamma(a) - std::lgamma(b) +
                       b * std::log1p(-x) + a * std::log(x);
  return 1.0 - std::exp(lback) / b / incbeta_fraction(b, a, 1.0 - x);
}

struct Density {
  int d;
  double a;      // (d - 1)/2
  double logc;   // log C_d
  explicit Density(int dim) : d(dim), a((dim - 1) / 2.0) {
    logc = std::lgamma(dim / 2.0) - std::lgamma((dim - 1) / 2.0) - 0.5 * std::log(M_PI);
  }
  // P(X > t) for t in [0, 1]: I_{(1 - t)/2}(a, a)
  // Only called for t in [0, 1]; P(X > 0) = 1/2 by symmetry.
  double tail(double t) const {
    if (t <= 0.0) return 0.5;
    return incbeta(a, a, 0.5 * (1.0 - t));
  }
  // F1(x) with dF1/dx = -x f_d(x)
  double f1(double x) const {
    const double u = 1.0 - x * x;
    if (u <= 0.0) return 0.0;
    return std::exp(logc + a * std::log(u)) / (d - 1);
  }
};

}  // namespace

extern "C" int tq_build_codebook(int head_dim, int bits, double *centroids,
                                 double *thresholds) {
  if (!centroids || !thresholds) return TQ_ERR_ARG;
  if (bits < TQ_MIN_BITS || bits > TQ_MAX_BITS) return TQ_ERR_BITS;
  if (head_dim < 2 || head_dim > 65536 || (head_dim & (head_dim - 1))) return TQ_ERR_HEAD_DIM;

  const int L = 1 << bits;
  const int h = L / 2;
  const Density f(head_dim);

  // Start: centroid i at the quantile (h + i + 1/2)/L, found by bisection on
  // the tail probability (tail is decreasing on [0, 1]).
  std::vector<double> p(h), next(h), edge(h + 1), mass(h);
  for (int i = 0; i < h; ++i) {
    const double want_tail = 1.0 - (h + i + 0.5) / L;
    double lo = 0.0, hi = 1.0;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (mid == lo || mid == hi) break;
      if (f.tail(mid) > want_tail) lo = mid; else hi = mid;
    }
    p[i] = 0.5 * (lo + hi);
  }

  // Fixed-point iteration; the same stopping rule as the reference
  // description: relative movement below 1e-13, or no new minimum of the
  // movement for 2000 steps (rounding floor), or 10^6 steps.
  const double tol = 1e-13;
  const int max_iter = 1000000, stall = 2000;
  double best = INFINITY;
  int since = 0;
  std::vector<double> tails(h + 1), f1s(h + 1);
  for (int it = 0; it < max_iter; ++it) {
    edge[0] = 0.0;
    for (int i = 1; i < h; ++i) edge[i] = 0.5 * (p[i - 1] + p[i]);
    edge[h] = 1.0;
    for (int i = 0; i <= h; ++i) {
      tails[i] = (i == 0) ? 0.5 : (i == h ? 0.0 : f.tail(edge[i]));
      f1s[i] = f.f1(edge[i]);
    }
    double moved = 0.0, top = 0.0;
    for (int i = 0; i < h; ++i) {
      next[i] = (f1s[i] - f1s[i + 1]) / (tails[i] - tails[i + 1]);
      moved = std::fmax(moved, std::fabs(next[i] - p[i]));
      top = std::fmax(top, std::fabs(next[i]));
    }
    p.swap(next);
    if (moved <= tol * top) break;
    if (moved < best) {
      best = moved;
      since = 0;
    } else if (++since >= stall) {
      break;
    }
  }

  for (int i = 0; i < h; ++i) {
    centroids[h + i] = p[i];
    centroids[h - 1 - i] = -p[i];
  }
  for (int k = 0; k + 1 < L; ++k) thresholds[k] = 0.5 * (centroids[k] + centroids[k + 1]);
  thresholds[h - 1] = 0.0;
  return TQ_OK;
}

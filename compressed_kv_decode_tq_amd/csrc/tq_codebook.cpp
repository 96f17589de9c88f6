// Lloyd-Max codebook for one coordinate of a randomly rotated unit vector,
// solved in double precision on the host.
//
// After a fixed random rotation every coordinate of a unit vector in R^d has
// the same law, a concentrated Beta-type law (page "TurboQuant — Random rotation
// trước khi quantize, 3-bit KV cache không mất accuracy", section "Ý tưởng cốt
// lõi"), so one MSE-optimal scalar quantizer serves every coordinate.  The
// density is f(x) = C (1 - x^2)^a on [-1, 1] with a = (d - 3) / 2.
//
// Cell integrals are exact: with J_a(x) = integral_0^x (1 - t^2)^a dt,
//   integration by parts gives J_a(x) = (x (1-x^2)^a + 2a J_{a-1}(x)) / (2a + 1),
//   started from J_0(x) = x or J_{1/2}(x) = (x sqrt(1-x^2) + asin x) / 2
//   (a is an integer or a half-integer for integer d); the recursion multiplies
//   earlier errors by 2a/(2a+1) < 1, so it is stable;
// and integral x (1-x^2)^a dx = -(1-x^2)^(a+1) / (2(a+1)).
// Lloyd's iteration (thresholds at midpoints, centroids at cell means) then
// converges to the unique optimum of this log-concave density.
#include <cmath>
#include <vector>

#include "tq_internal.h"

namespace tq {
namespace {

// J_a(x) for x in [0, 1], a = (d - 3) / 2.
double half_integral(double x, int d) {
  const double w = 1.0 - x * x;
  double j, a, wa;  // J_a(x), a, w^a
  if ((d - 3) % 2 == 0) {  // integer exponent
    j = x;
    a = 0.0;
    wa = 1.0;
  } else {                 // half-integer exponent
    wa = std::sqrt(w);
    j = 0.5 * (x * wa + std::asin(x));
    a = 0.5;
  }
  const double a_end = 0.5 * (d - 3);
  while (a < a_end - 0.25) {
    a += 1.0;
    wa *= w;
    j = (x * wa + 2.0 * a * j) / (2.0 * a + 1.0);
  }
  return j;
}

// Signed integral of (1 - t^2)^a from 0 to x.
double signed_integral(double x, int d) {
  return x >= 0 ? half_integral(x, d) : -half_integral(-x, d);
}

// Unnormalised first moment antiderivative: -(1 - x^2)^(a+1) / (2(a+1)).
double moment_anti(double x, int d) {
  const double a1 = 0.5 * (d - 3) + 1.0;
  return -std::pow(1.0 - x * x, a1) / (2.0 * a1);
}

}  // namespace

int make_codebook(int d, int bits, double* cent, double* thr) {
  const int levels = 1 << bits;
  // start from equal-width cells over +-3 standard deviations (std = 1/sqrt(d)),
  // kept inside the support [-1, 1]: for d < 10 three deviations reach past it,
  // and a midpoint beyond +-1 has no defined cell integral
  std::vector<double> c(levels), cn(levels), e(levels + 1);
  const double span = std::fmin(3.0 / std::sqrt(static_cast<double>(d)), 1.0);
  for (int k = 0; k < levels; ++k) c[k] = -span + span * (2.0 * k + 1.0) / levels;
  for (int it = 0; it < 200000; ++it) {
    e[0] = -1.0;
    e[levels] = 1.0;
    for (int k = 1; k < levels; ++k) e[k] = 0.5 * (c[k - 1] + c[k]);
    double moved = 0.0;
    for (int k = 0; k < levels; ++k) {
      // use the symmetric cell in the lower half so that both halves are
      // computed from identical numbers and the table stays exactly symmetric
      if (k >= levels / 2) {
        cn[k] = -cn[levels - 1 - k];
        continue;
      }
      const double m0 = signed_integral(e[k + 1], d) - signed_integral(e[k], d);
      const double m1 = moment_anti(e[k + 1], d) - moment_anti(e[k], d);
      cn[k] = m1 / m0;
    }
    for (int k = 0; k < levels; ++k) moved = std::fmax(moved, std::fabs(cn[k] - c[k]));
    c.swap(cn);
    if (moved < 1e-15) break;
  }
  for (int k = 0; k < levels; ++k) cent[k] = c[k];
  for (int k = 0; k + 1 < levels; ++k) thr[k] = 0.5 * (c[k] + c[k + 1]);
  if (levels >= 2) thr[levels / 2 - 1] = 0.0;  // exact middle of a symmetric table
  return TQ_OK;
}

// Walsh-Hadamard expansion of a codebook over the bits of its index.  With
// x_k = 2 b_k - 1, any table is c[idx] = sum_S a_S prod_{k in S} x_k, with
// a_S = 2^-b sum_idx c[idx] prod_{k in S} x_k(idx).  An antisymmetric table
// (c[2^b-1-i] = -c[i], as every Lloyd-Max table of a symmetric law is) has
// a_S = 0 for every even |S|, and for odd |S| the product is 2 par_S - 1
// (par_S = XOR of the bits in S), so c[idx] = -sum a_S + sum 2 a_S par_S.
int plane_expansion(const float* cent, int bits, float* w, float* cst) {
  if (bits < 1 || bits > 3) return 0;
  const int levels = 1 << bits;
  double amax = 0.0;
  for (int i = 0; i < levels; ++i) amax = std::fmax(amax, std::fabs((double)cent[i]));
  for (int i = 0; i < levels; ++i)
    if (std::fabs((double)cent[i] + (double)cent[levels - 1 - i]) > 1e-6 * amax) return 0;
  // odd subsets in plane order: {0}, {1}, {2}, {0,1,2}
  const int subsets[4] = {1, 2, 4, 7};
  const int planes = 1 << (bits - 1);
  double c0 = 0.0;
  for (int p = 0; p < planes; ++p) {
    const int s = subsets[p];
    double acc = 0.0;
    for (int idx = 0; idx < levels; ++idx) {
      double prod = 1.0;
      for (int k = 0; k < bits; ++k)
        if (s & (1 << k)) prod *= ((idx >> k) & 1) ? 1.0 : -1.0;
      acc += (double)cent[idx] * prod;
    }
    const double a = acc / levels;
    w[p] = (float)(2.0 * a);
    c0 -= a;
  }
  *cst = (float)c0;
  return planes;
}

}  // namespace tq

// Lloyd-Max activation codebook (host code): the levels of the minimum-MSE
// 2^b-level scalar quantizer for one coordinate of a rotated token.
//
// OrbitQuant PR #25, "Default changes": Lloyd-Max codes are the activation
// quantizer below 8 bits; codebooks are built per width d, by a Newton solver
// (about 0.1 s per width up to d = 30720 for 8-bit tables).  CentriQ Sec. 2
// ("Related work"): the codebook is derived from the post-rotation marginal.
//
// Marginal: one coordinate T of a point uniform on the unit sphere S^{d-1},
// density (1 - t^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1]; tokens are
// normalised by their RMS, so the levels are for U = sqrt(d) T (variance 1).
// With n = (d - 1) / 2:
//   P(0 <= U <= u) = I_x(1/2, n) / 2,  x = u^2 / d   (T^2 ~ Beta(1/2, n))
//   int u g(u) du  = -sqrt(d) (1 - u^2/d)^n / ((d - 1) B(1/2, n))
// The marginal is even, so only the positive half is solved: boundaries
// 0 = p_0 < p_1 < ... < p_{h-1} < p_h = sqrt(d) (h = 2^(b-1)), levels
// c_i = E[U | p_i < U <= p_{i+1}], and Lloyd's conditions
//   F_j = p_j - (c_{j-1} + c_j) / 2 = 0,   j = 1 .. h-1.
// The Jacobian is tridiagonal: dc_i/dp_i = g(p_i)(c_i - p_i)/P_i and
// dc_i/dp_{i+1} = g(p_{i+1})(p_{i+1} - c_i)/P_i.  Start: boundaries at equal
// probabilities (bisection), a few Lloyd sweeps, then damped Newton steps.
//
// I_x(a, b) is evaluated from its continued fraction (Abramowitz & Stegun
// 26.5.8) by the modified Lentz method, on the side of the symmetry
// I_x(a, b) = 1 - I_{1-x}(b, a) where the fraction converges fast; both the
// value and its complement are returned so that small tail masses keep their
// relative accuracy.
#include <cmath>
#include <vector>

#include "oq_internal.h"

namespace oq {
namespace {

// x^a (1 - x)^b / (a B(a, b)) times the continued fraction 1 / (1 + d1 / (1 + d2 / ...));
// ln x and ln(1 - x) come from the caller, each from its accurate form
double ibeta_cf(double a, double b, double x, double lnx, double ln1mx, double log_beta) {
  const double tiny = 1e-300;
  double f = 1.0, C = 1.0, D = 0.0;
  for (int m2 = 1; m2 < 20000; ++m2) {
    const int m = m2 / 2;
    double dm;
    if (m2 & 1)
      dm = -(a + m) * (a + b + m) * x / ((a + 2 * m) * (a + 2 * m + 1));
    else
      dm = m * (b - m) * x / ((a + 2 * m - 1) * (a + 2 * m));
    D = 1.0 + dm * D;
    if (std::fabs(D) < tiny) D = tiny;
    D = 1.0 / D;
    C = 1.0 + dm / C;
    if (std::fabs(C) < tiny) C = tiny;
    const double delta = C * D;
    f *= delta;
    if (std::fabs(delta - 1.0) < 1e-16) break;
  }
  const double pre = std::exp(a * lnx + b * ln1mx - std::log(a) - log_beta);
  return pre / f;
}

struct Marginal {
  int d;
  double n, sd, log_beta, moment_norm, dens_norm;

  explicit Marginal(int d_) : d(d_), n((d_ - 1) / 2.0), sd(std::sqrt((double)d_)) {
    // B(1/2, n) = sqrt(pi) Gamma(n) / Gamma(n + 1/2); the ratio
    // R(n) = Gamma(n + 1/2) / Gamma(n) by the recurrence R(n + 1) = R(n) (n + 1/2) / n
    // from R(1) = sqrt(pi) / 2 (integer n) or R(1/2) = 1 / sqrt(pi)
    const double spi = std::sqrt(M_PI);
    double R, k;
    if (std::fmod(n, 1.0) == 0.0) {
      R = spi / 2;
      k = 1.0;
    } else {
      R = 1.0 / spi;
      k = 0.5;
    }
    for (; k < n - 0.25; k += 1.0) R *= (k + 0.5) / k;
    log_beta = std::log(spi / R);
    moment_norm = sd / ((d - 1) * std::exp(log_beta));
    dens_norm = 1.0 / (sd * std::exp(log_beta));
  }
  // I_x(1/2, n) and 1 - I_x(1/2, n) for x = u^2 / d
  void ibeta(double u, double *I, double *Ic) const {
    double x = (u / sd) * (u / sd);
    if (x <= 0.0) {
      *I = 0.0;
      *Ic = 1.0;
      return;
    }
    if (x >= 1.0) {
      *I = 1.0;
      *Ic = 0.0;
      return;
    }
    const double a = 0.5, b = n;
    if (x < (a + 1.0) / (a + b + 2.0)) {
      *I = ibeta_cf(a, b, x, std::log(x), std::log1p(-x), log_beta);
      *Ic = 1.0 - *I;
    } else {
      *Ic = ibeta_cf(b, a, 1.0 - x, std::log1p(-x), std::log(x), log_beta);
      *I = 1.0 - *Ic;
    }
  }
  // P(a < U <= b), 0 <= a < b, from whichever form is small
  double mass(double a, double b) const {
    double Ia, Ica, Ib, Icb;
    ibeta(a, &Ia, &Ica);
    ibeta(b, &Ib, &Icb);
    return Ia < 0.5 ? 0.5 * (Ib - Ia) : 0.5 * (Ica - Icb);
  }
  // int_a^b u g(u) du with E(u) = (1 - u^2/d)^n differenced without cancellation
  double moment(double a, double b) const {
    const double xa = n * std::log1p(-std::min((a / sd) * (a / sd), 1.0));
    const double tb = std::min((b / sd) * (b / sd), 1.0);
    if (tb >= 1.0) return moment_norm * std::exp(xa);
    const double xb = n * std::log1p(-tb);
    return moment_norm * std::exp(xb) * std::expm1(xa - xb);
  }
  double density(double u) const {
    const double t = std::min((u / sd) * (u / sd), 1.0);
    if (t >= 1.0) return 0.0;
    return dens_norm * std::exp((d - 3) / 2.0 * std::log1p(-t));
  }
  double upper_tail(double u) const {  // P(U > u), u >= 0
    double I, Ic;
    ibeta(u, &I, &Ic);
    return 0.5 * Ic;
  }
};

// centroids c[0..h-1] of the cells [p_i, p_{i+1}] (p_0 = 0, p_h = sqrt d), masses P
void half_centroids(const Marginal &g, const std::vector<double> &p, std::vector<double> &c, std::vector<double> &P) {
  const int h = (int)p.size() + 1;
  c.resize(h);
  P.resize(h);
  for (int i = 0; i < h; ++i) {
    const double lo = i == 0 ? 0.0 : p[i - 1];
    const double hi = i == h - 1 ? g.sd : p[i];
    P[i] = g.mass(lo, hi);
    c[i] = g.moment(lo, hi) / P[i];
  }
}

double residual(const Marginal &g, const std::vector<double> &p, std::vector<double> &F, std::vector<double> &c,
                std::vector<double> &P) {
  half_centroids(g, p, c, P);
  double mx = 0.0;
  F.resize(p.size());
  for (size_t j = 0; j < p.size(); ++j) {
    F[j] = p[j] - 0.5 * (c[j] + c[j + 1]);
    if (!std::isfinite(F[j])) return INFINITY;
    mx = std::max(mx, std::fabs(F[j]));
  }
  return mx;
}

bool increasing(const Marginal &g, const std::vector<double> &p) {
  double prev = 0.0;
  for (double v : p) {
    if (!(v > prev)) return false;
    prev = v;
  }
  return prev < g.sd;
}

}  // namespace

double lloyd_max_solve(int d, int bits, double *levels) {
  if (d < 3 || bits < 1 || bits > 8) return -1.0;
  const Marginal g(d);
  const int L = 1 << bits, h = L / 2;
  std::vector<double> p(h - 1), c, P, F;
  // boundaries at P(U > p_j) = (h - j) / L, by bisection on the upper tail
  for (int j = 1; j < h; ++j) {
    const double target = (double)(h - j) / L;
    double lo = 0.0, hi = g.sd;
    for (int it = 0; it < 200; ++it) {
      const double mid = 0.5 * (lo + hi);
      if (mid <= lo || mid >= hi) break;
      if (g.upper_tail(mid) > target)
        lo = mid;
      else
        hi = mid;
    }
    p[j - 1] = 0.5 * (lo + hi);
  }
  for (int it = 0; it < 40 && h > 1; ++it) {
    half_centroids(g, p, c, P);
    for (int j = 0; j < h - 1; ++j) p[j] = 0.5 * (c[j] + c[j + 1]);
  }
  double res = h > 1 ? residual(g, p, F, c, P) : 0.0;
  std::vector<double> lo_d(h), di(h), up_d(h), step(h), pn(h), Fn, cn, Pn;
  for (int it = 0; it < 200 && h > 1 && res > 0.0; ++it) {
    const int m = h - 1;
    // tridiagonal Jacobian of F at p (index j = 0 .. m-1 is boundary p_{j+1})
    for (int j = 0; j < m; ++j) {
      const double pj = p[j], gj = g.density(pj);
      di[j] = 1.0 - 0.5 * (gj * (pj - c[j]) / P[j] + gj * (c[j + 1] - pj) / P[j + 1]);
      lo_d[j] = j > 0 ? -0.5 * g.density(p[j - 1]) * (c[j] - p[j - 1]) / P[j] : 0.0;
      up_d[j] = j < m - 1 ? -0.5 * g.density(p[j + 1]) * (p[j + 1] - c[j + 1]) / P[j + 1] : 0.0;
      step[j] = -F[j];
    }
    // Thomas solve
    for (int j = 1; j < m; ++j) {
      const double w = lo_d[j] / di[j - 1];
      di[j] -= w * up_d[j - 1];
      step[j] -= w * step[j - 1];
    }
    step[m - 1] /= di[m - 1];
    for (int j = m - 2; j >= 0; --j) step[j] = (step[j] - up_d[j] * step[j + 1]) / di[j];
    double alpha = 1.0, rn = INFINITY;
    pn.resize(m);
    for (int k = 0; k < 40; ++k, alpha *= 0.5) {
      for (int j = 0; j < m; ++j) pn[j] = p[j] + alpha * step[j];
      if (!increasing(g, pn)) continue;
      rn = residual(g, pn, Fn, cn, Pn);
      if (rn < res) break;
    }
    if (!(rn < res)) break;  // no further progress: converged to rounding level
    p.swap(pn);
    F.swap(Fn);
    c.swap(cn);
    P.swap(Pn);
    res = rn;
  }
  if (h == 1) half_centroids(g, p, c, P);
  for (int i = 0; i < h; ++i) {
    levels[h + i] = c[i];
    levels[h - 1 - i] = -c[i];
  }
  return res;
}

}  // namespace oq

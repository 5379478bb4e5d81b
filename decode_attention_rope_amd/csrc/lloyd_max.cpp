// Frozen Gaussian Lloyd-Max tables used by the kernels.
//
// TurboQuant-MSE (named as the base quantizer in "RoPE-Aware Bit Allocation
// for KV-Cache Quantization", abstract) codes each rotated, rescaled
// coordinate with the minimum-MSE scalar quantizer of N(0, 1).  The b-bit
// quantizer has 2^b cells; its decision levels lie halfway between adjacent
// reconstruction levels and every reconstruction level is the mean of N(0, 1)
// over its cell.  D(b) is its mean squared error (D(0) = 1: nothing coded).
//
// The quantizer is odd-symmetric, so only the K = 2^(b-1) cells on the
// positive axis are solved for.  Unknowns: the positive decision levels
// u_1 < ... < u_{K-1} (u_0 = 0, u_K = +inf).  Residual
//     F_k(u) = u_k - (y_k + y_{k+1}) / 2,     y_k = mean of N(0,1) on (u_{k-1}, u_k),
// solved by Newton's method (the Jacobian is tridiagonal) from the Panter-Dite
// high-rate point density, whose cell edges are sqrt(3) times Gaussian
// quantiles.  All arithmetic is fp64; the tables are then rounded to fp32.

#include <cmath>
#include <cstring>
#include <utility>
#include <vector>

#include "bgtq_internal.h"

namespace bgtq {
namespace {

constexpr double kInvSqrt2Pi = 0.39894228040143267794;
constexpr double kInvSqrt2 = 0.70710678118654752440;

double density(double x) { return std::isinf(x) ? 0.0 : kInvSqrt2Pi * std::exp(-0.5 * x * x); }

// Upper tail Q(x) = P(X > x).
double upper_tail(double x) { return std::isinf(x) ? 0.0 : 0.5 * std::erfc(x * kInvSqrt2); }

// x with Q(x) = q, for 0 < q < 1/2, by bisection on the monotone tail.
double tail_inverse(double q) {
  double lo = 0.0, hi = 40.0;
  for (int it = 0; it < 200; ++it) {
    double mid = 0.5 * (lo + hi);
    if (upper_tail(mid) > q) lo = mid; else hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct Cell { double mean, mass; };

// Mean and probability of N(0,1) on (a, b) with 0 <= a < b <= inf.
Cell positive_cell(double a, double b) {
  double mass = upper_tail(a) - upper_tail(b);
  return {(density(a) - density(b)) / mass, mass};
}

// Solve the positive half; returns decision levels u[0..K] (u[0] = 0, u[K] = inf)
// and reconstruction levels y[1..K] (y[0] unused).
void solve_half(int bits, std::vector<double>& u, std::vector<double>& y, std::vector<double>& p) {
  const int K = 1 << (bits - 1);
  u.assign(K + 1, 0.0);
  u[K] = INFINITY;
  for (int k = 1; k < K; ++k) {
    // Panter-Dite: the positive edge k sits at sqrt(3) * Phi^{-1}(1/2 + k/(2K)).
    u[k] = std::sqrt(3.0) * tail_inverse(0.5 - 0.5 * double(k) / double(K));
  }
  y.assign(K + 1, 0.0);
  p.assign(K + 1, 0.0);
  const int n = K - 1;  // unknowns u_1..u_{K-1}
  std::vector<double> f(n), diag(n), sub(n), sup(n), cp(n), dp(n);
  for (int iter = 0; iter < 200 && n > 0; ++iter) {
    for (int k = 1; k <= K; ++k) {
      Cell c = positive_cell(u[k - 1], u[k]);
      y[k] = c.mean;
      p[k] = c.mass;
    }
    for (int r = 0; r < n; ++r) {
      const int k = r + 1;           // unknown u_k
      const double uk = u[k];
      f[r] = uk - 0.5 * (y[k] + y[k + 1]);
      // d y_k / d u_k (upper edge of cell k) and d y_{k+1} / d u_k (lower edge of cell k+1)
      const double dyk = density(uk) * (uk - y[k]) / p[k];
      const double dyk1 = density(uk) * (y[k + 1] - uk) / p[k + 1];
      diag[r] = 1.0 - 0.5 * (dyk + dyk1);
      // d F_k / d u_{k-1}: through y_k's lower edge
      sub[r] = (k >= 2) ? -0.5 * density(u[k - 1]) * (y[k] - u[k - 1]) / p[k] : 0.0;
      // d F_k / d u_{k+1}: through y_{k+1}'s upper edge
      sup[r] = (k + 1 <= K - 1) ? -0.5 * density(u[k + 1]) * (u[k + 1] - y[k + 1]) / p[k + 1] : 0.0;
    }
    // Thomas algorithm for the tridiagonal system J * delta = f.
    cp[0] = sup[0] / diag[0];
    dp[0] = f[0] / diag[0];
    for (int r = 1; r < n; ++r) {
      const double den = diag[r] - sub[r] * cp[r - 1];
      cp[r] = sup[r] / den;
      dp[r] = (f[r] - sub[r] * dp[r - 1]) / den;
    }
    double step_max = 0.0;
    for (int r = n - 1; r >= 0; --r) {
      const double delta = dp[r] - ((r + 1 < n) ? cp[r] * dp[r + 1] : 0.0);
      dp[r] = delta;
      u[r + 1] -= delta;
      step_max = std::fmax(step_max, std::fabs(delta));
    }
    if (step_max < 1e-15) break;
  }
  for (int k = 1; k <= K; ++k) {
    Cell c = positive_cell(u[k - 1], u[k]);
    y[k] = c.mean;
    p[k] = c.mass;
  }
}

Tables build_tables() {
  Tables t{};
  t.dist[0] = 1.0;
  for (int bits = 1; bits <= kMaxBits; ++bits) {
    std::vector<double> u, y, p;
    solve_half(bits, u, y, p);
    const int K = 1 << (bits - 1), N = 2 * K;
    // decision levels, ascending: -u_{K-1}..-u_1, 0, u_1..u_{K-1}
    for (int k = 1; k < K; ++k) {
      t.thr[bits - 1][K - 1 + k] = float(u[k]);
      t.thr[bits - 1][K - 1 - k] = -float(u[k]);
    }
    t.thr[bits - 1][K - 1] = 0.0f;
    // reconstruction levels, ascending: -y_K..-y_1, y_1..y_K
    for (int k = 1; k <= K; ++k) {
      t.cen[bits - 1][K - 1 + k] = float(y[k]);
      t.cen[bits - 1][K - k] = -float(y[k]);
    }
    double second_moment = 0.0;
    for (int k = 1; k <= K; ++k) second_moment += y[k] * y[k] * p[k];
    t.dist[bits] = double(float(1.0 - 2.0 * second_moment));
    (void)N;
  }
  for (int b = 0; b < kMaxBits; ++b) t.dgain[b] = t.dist[b] - t.dist[b + 1];
  // fp16 decoder tables (round to nearest even from the fp32 levels)
  auto h16 = [](float x) { const _Float16 h = (_Float16)x; uint16_t u; std::memcpy(&u, &h, 2); return u; };
  for (int w = 1; w <= 5; ++w) {
    const int base = ((1 << (2 * w)) - 4) / 3;
    for (int idx = 0; idx < (1 << (2 * w)); ++idx) {
      const int c0 = idx & ((1 << w) - 1), c1 = idx >> w;
      t.pair[base + idx] = uint32_t(h16(t.cen[w - 1][c0])) | uint32_t(h16(t.cen[w - 1][c1])) << 16;
    }
  }
  for (int w = 1; w <= 8; ++w) {
    const int base = (1 << w) - 2;
    for (int c = 0; c < (1 << w); ++c) t.single[base + c] = h16(t.cen[w - 1][c]);
  }
  // hi + lo: the remainder cen - hi is exact in fp32 (hi is cen rounded to 11 bits), then rounded
  // to fp16 once more
  auto hl = [&](int w, int c) {
    const float x = t.cen[w - 1][c];
    const uint16_t hi = h16(x);
    _Float16 hf;
    std::memcpy(&hf, &hi, 2);
    return std::pair<uint16_t, uint16_t>(hi, h16(x - float(hf)));
  };
  for (int w = 1; w <= 5; ++w) {
    const int base = ((1 << (2 * w)) - 4) / 3;
    for (int idx = 0; idx < (1 << (2 * w)); ++idx) {
      const auto a = hl(w, idx & ((1 << w) - 1)), b = hl(w, idx >> w);
      t.pair_hl[base + idx][0] = uint32_t(a.first) | uint32_t(b.first) << 16;
      t.pair_hl[base + idx][1] = uint32_t(a.second) | uint32_t(b.second) << 16;
    }
  }
  for (int w = 1; w <= 8; ++w) {
    const int base = (1 << w) - 2;
    for (int c = 0; c < (1 << w); ++c) {
      const auto a = hl(w, c);
      t.single_hl[base + c] = uint32_t(a.first) | uint32_t(a.second) << 16;
    }
  }
  return t;
}

}  // namespace

const Tables& host_tables() {
  static const Tables tables = build_tables();
  return tables;
}

}  // namespace bgtq

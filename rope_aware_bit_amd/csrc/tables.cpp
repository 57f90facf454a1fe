// Constant tables of the quantizers, built once on the host when a cache is created.
//
// TQ-MSE-style codebooks (RoPE-Aware Bit Allocation for KV-Cache Quantization,
// abstract: the quantizer derives from TurboQuant-MSE).  Reading: the
// 2^b-level MSE-optimal scalar quantizer of a standard normal (no rotation),
// centroids rounded once from fp64 to fp16 (nearest-even); boundaries are the
// fp32 rounding of the exact midpoint of neighbouring fp16 centroids.
//
// Greedy gains: delta(b) = fp32(c(b) - c(b+1)) with c(b) the exact N(0,1)
// mean squared error of the b-bit fp16 codebook and c(0) = 1.
//
// 16-level Gaussian-quantile codebook (NQKV review, "What carries the
// argument"): levels Phi^-1((k + 1/2)/16) / Phi^-1(31/32), fp16; fp32 midpoint
// boundaries.
//
// The optimum is found by Newton's method on the positive half of the
// symmetric quantizer (a tridiagonal system solved by forward elimination).
#include <cmath>
#include <cstring>
#include <limits>
#include <vector>

#include "kvq_internal.h"

namespace kvq {
namespace {

const double kInvSqrt2 = 0.70710678118654752440;
const double kInvSqrt2Pi = 0.39894228040143267794;

double tail(double x) {  // P(Z > x)
  if (std::isinf(x)) return x > 0 ? 0.0 : 1.0;
  return 0.5 * std::erfc(x * kInvSqrt2);
}

double pdf(double x) {
  if (std::isinf(x)) return 0.0;
  return kInvSqrt2Pi * std::exp(-0.5 * x * x);
}

// P(a < Z <= b) for 0 <= a < b (upper tails keep precision on the positive half)
double mass_pos(double a, double b) { return tail(a) - tail(b); }

double normal_cdf(double x) { return x >= 0 ? 1.0 - tail(x) : tail(-x); }

// Standard normal quantile: bisection on the distribution function, then Newton polish.
double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p) lo = mid; else hi = mid;
  }
  double x = 0.5 * (lo + hi);
  for (int i = 0; i < 3; ++i) x -= (normal_cdf(x) - p) / pdf(x);
  return x;
}

// Positive-half centroids of the 2n-level optimum (ascending), by Newton.
std::vector<double> lloyd_max_positive(int n) {
  std::vector<double> c(n), F(n), diag(n), sub(n), sup(n), step(n);
  const int L = 2 * n;
  for (int k = 0; k < n; ++k) c[k] = normal_quantile((n + k + 0.5) / L);
  for (int it = 0; it < 200; ++it) {
    double maxstep = 0.0;
    for (int k = 0; k < n; ++k) {
      double lo = k == 0 ? 0.0 : 0.5 * (c[k - 1] + c[k]);
      double hi = k == n - 1 ? std::numeric_limits<double>::infinity() : 0.5 * (c[k] + c[k + 1]);
      double P = mass_pos(lo, hi);
      double mu = (pdf(lo) - pdf(hi)) / P;
      F[k] = mu - c[k];
      diag[k] = -1.0;
      sub[k] = sup[k] = 0.0;
      if (k > 0) {
        double d = 0.5 * pdf(lo) * (mu - lo) / P;
        sub[k] = d;
        diag[k] += d;
      }
      if (k < n - 1) {
        double d = 0.5 * pdf(hi) * (hi - mu) / P;
        sup[k] = d;
        diag[k] += d;
      }
    }
    // solve J step = -F (tridiagonal: sub, diag, sup)
    std::vector<double> cp(n), dp(n);
    cp[0] = sup[0] / diag[0];
    dp[0] = -F[0] / diag[0];
    for (int k = 1; k < n; ++k) {
      double m = diag[k] - sub[k] * cp[k - 1];
      cp[k] = sup[k] / m;
      dp[k] = (-F[k] - sub[k] * dp[k - 1]) / m;
    }
    step[n - 1] = dp[n - 1];
    for (int k = n - 2; k >= 0; --k) step[k] = dp[k] - cp[k] * step[k + 1];
    for (int k = 0; k < n; ++k) {
      c[k] += step[k];
      maxstep = std::fmax(maxstep, std::fabs(step[k]));
    }
    if (maxstep < 1e-15) break;
  }
  return c;
}

// fp64 -> fp16 bit pattern, one round-to-nearest-even rounding (finite inputs).
uint16_t half_bits(double x) {
  uint16_t sign = std::signbit(x) ? 0x8000 : 0;
  double a = std::fabs(x);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);  // a = m * 2^e, m in [0.5, 1)
  e -= 1;             // a = m' * 2^e, m' in [1, 2)
  if (e < -14) {      // subnormal: multiples of 2^-24
    double q = std::nearbyint(std::ldexp(a, 24));
    return sign | static_cast<uint16_t>(q);  // q == 1024 lands on the smallest normal
  }
  double q = std::nearbyint(std::ldexp(a, 10 - e));  // in [1024, 2048]
  if (q == 2048.0) { q = 1024.0; ++e; }
  if (e > 15) return sign | 0x7C00;
  return sign | static_cast<uint16_t>(((e + 15) << 10) | (static_cast<int>(q) - 1024));
}

double half_value(uint16_t h) {
  int e = (h >> 10) & 0x1F, m = h & 0x3FF;
  double v = e == 0 ? std::ldexp(static_cast<double>(m), -24)
                    : std::ldexp(static_cast<double>(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

// exact N(0,1) MSE of a symmetric quantizer given by its positive half
double symmetric_mse(const std::vector<double>& cpos, const std::vector<double>& bpos) {
  // cells [bpos[k-1], bpos[k]) with bpos[-1] = 0 and bpos[n-1] = +inf
  const int n = static_cast<int>(cpos.size());
  double sum = 0.0;
  for (int k = 0; k < n; ++k) {
    double a = k == 0 ? 0.0 : bpos[k - 1];
    double b = k == n - 1 ? std::numeric_limits<double>::infinity() : bpos[k];
    double P = mass_pos(a, b);
    double pa = pdf(a), pb = pdf(b);
    double ta = a * pa, tb = std::isinf(b) ? 0.0 : b * pb;
    sum += (1.0 + cpos[k] * cpos[k]) * P - 2.0 * cpos[k] * (pa - pb) + (ta - tb);
  }
  return 2.0 * sum;
}

}  // namespace

void build_tables(Tables* t) {
  std::memset(t, 0, sizeof(Tables));
  const float inf = std::numeric_limits<float>::infinity();
  double c[kMaxBits + 1];
  c[0] = 1.0;
  for (int k = 0; k < 256; ++k) t->bd[0][k] = inf;   // width 0: no boundary, every search stays at code 0
  for (int b = 1; b <= kMaxBits; ++b) {
    const int n = 1 << (b - 1), L = 1 << b;
    std::vector<double> cpos = lloyd_max_positive(n);
    std::vector<double> hpos(n), bpos(n);
    for (int k = 0; k < n; ++k) {
      uint16_t h = half_bits(cpos[k]);
      hpos[k] = half_value(h);
      t->cb[b][n + k] = h;
      t->cb[b][n - 1 - k] = h | 0x8000;
    }
    for (int k = 0; k < 256; ++k) t->bd[b][k] = inf;   // +inf after the 2^b - 1 boundaries
    t->bd[b][n - 1] = 0.0f;
    for (int k = 0; k + 1 < n; ++k) {
      float m = static_cast<float>(0.5 * (hpos[k] + hpos[k + 1]));  // exact midpoint, one rounding
      bpos[k] = m;
      t->bd[b][n + k] = m;
      t->bd[b][n - 2 - k] = -m;
    }
    c[b] = symmetric_mse(hpos, bpos);
  }
  for (int b = 0; b < kMaxBits; ++b) t->delta[b] = static_cast<float>(c[b] - c[b + 1]);

  const double zs = normal_quantile(31.0 / 32.0);
  double lv[16];
  for (int k = 8; k < 16; ++k) {
    double v = normal_quantile((k + 0.5) / 16.0) / zs;
    uint16_t h = half_bits(v);
    lv[k] = half_value(h);
    lv[15 - k] = -lv[k];
    t->nf_cb[k] = h;
    t->nf_cb[15 - k] = h | 0x8000;
  }
  for (int k = 0; k < 15; ++k) t->nf_bd[k] = static_cast<float>(0.5 * (lv[k] + lv[k + 1]));
  t->nf_bd[15] = inf;

  uint16_t ints[256];   // fp16 bit patterns of the integers 0 .. 255
  for (int k = 0; k < 256; ++k) ints[k] = half_bits(static_cast<double>(k));
  for (int img = 0; img < 3; ++img) {
    uint8_t* out = t->lds_image[img];
    for (int w = 1; w <= kMaxBits; ++w) {
      const uint16_t* cb = img == 2 ? ints : (img == 1 && w == 4) ? t->nf_cb : t->cb[w];
      for (int c = 0; c < (1 << w); ++c)
        std::memcpy(out + single_table_base(w) + 2 * c, &cb[c], 2);
      if (w <= 4) {
        for (int e = 0; e < (1 << (2 * w)); ++e) {
          const uint32_t v = static_cast<uint32_t>(cb[e & ((1 << w) - 1)]) |
                             (static_cast<uint32_t>(cb[e >> w]) << 16);
          std::memcpy(out + pair_table_base(w) + 4 * e, &v, 4);
        }
      }
    }
  }
}

}  // namespace kvq

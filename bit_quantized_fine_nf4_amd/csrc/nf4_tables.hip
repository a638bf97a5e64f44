// Host-side construction of the NF4 codebook and the encoder's bucket table.
//
// Codebook ([MC] "1. NormalFloat", [TT] §5 "NF4", [GO] "Idea one"): 16 values
// placed at quantiles of a standard normal, normalised to [-1, 1].  Reading
// used here (the pages give no formula): 8 positive quantiles at
// probabilities 1/2 + (d - 1/2) k/8, k = 1..8, 7 negative ones mirrored from
// 1/2 + (d - 1/2) k/7, k = 1..7, plus an exact zero, all divided by the
// quantile at d, where d = (31/32 + 29/30)/2 keeps the outermost quantile
// finite.  The quantiles are evaluated here in long double by bisection on the
// normal CDF written with erfc, then rounded once to float32.
//
// Encoder ([TT] §2 "Choose a scale, then round"): the code of a normalised
// value x = fp32(w / absmax) is the number of level midpoints strictly below
// x (nearest level, ties to the lower one).  The GPU evaluates
// y = fma(w, 16 * rcp(absmax), 16) instead of the division; |y - (16x + 16)|
// is bounded (see kGuard), so a bucket table over floor(y) decides the code
// except inside a narrow guard band around each midpoint, where the kernel
// falls back to the exact IEEE division.

#include <cfloat>
#include <cmath>
#include <mutex>

#include "common.h"

namespace ql {

namespace {

// |y - (16 x + 16)| <= 16 * 2^-22 (a 2-ulp reciprocal) + 2^-20 (fma rounding, y < 32)
// + 2^-21 (rounding of x itself) = 5.2e-6; use a margin of 1.5x.
constexpr double kGuard = 8e-6;

long double norm_cdf(long double x) { return 0.5L * erfcl(-x / sqrtl(2.0L)); }

long double norm_quantile(long double p) {
  long double lo = -40.0L, hi = 40.0L;
  for (int i = 0; i < 256; ++i) {
    long double mid = 0.5L * (lo + hi);
    if (norm_cdf(mid) < p) lo = mid; else hi = mid;
    if (!(hi - lo > 0)) break;
  }
  return 0.5L * (lo + hi);
}

float round_down_f32(double v) {
  float f = (float)v;
  if ((double)f > v) f = nextafterf(f, -INFINITY);
  return f;
}
float round_up_f32(double v) {
  float f = (float)v;
  if ((double)f < v) f = nextafterf(f, INFINITY);
  return f;
}

bool build(Nf4Tables &t) {
  const long double d = 0.5L * (31.0L / 32.0L + 29.0L / 30.0L);
  const long double top = norm_quantile(d);
  long double v[16];
  int k = 0;
  for (int i = 7; i >= 1; --i) v[k++] = -norm_quantile(0.5L + (d - 0.5L) * i / 7.0L) / top;
  v[k++] = 0.0L;
  for (int i = 1; i <= 8; ++i) v[k++] = norm_quantile(0.5L + (d - 0.5L) * i / 8.0L) / top;
  for (int i = 0; i < 16; ++i) t.level[i] = (float)v[i];
  t.level[0] = (float)(-norm_quantile(d) / top);  // exactly -1 by construction
  t.level[7] = 0.0f;
  for (int i = 1; i < 16; ++i)
    if (!(t.level[i] > t.level[i - 1])) return false;
  if (t.level[0] != -1.0f || t.level[15] != 1.0f) return false;

  double ymid[15];
  for (int j = 0; j < 15; ++j) {
    double m = ((double)t.level[j] + (double)t.level[j + 1]) * 0.5;  // exact in double
    t.thr[j] = round_down_f32(m);
    ymid[j] = 16.0 * m + 16.0;                                         // exact in double
  }
  for (int b = 0; b < kBuckets; ++b) {
    EncBucket &e = t.bucket[b];
    uint32_t below = 0;
    int inside = -1, count = 0;
    for (int j = 0; j < 15; ++j) {
      if (ymid[j] < (double)b) ++below;
      if (ymid[j] >= (double)b && ymid[j] < (double)(b + 1)) { inside = j; ++count; }
      // a guard band must never straddle a bucket edge
      if (fabs(ymid[j] - (double)b) <= kGuard) return false;
    }
    if (count > 1) return false;
    e.base = below;
    if (inside < 0) {
      e.hi = INFINITY;
      e.lo = INFINITY;
      e.tx = INFINITY;
    } else {
      e.hi = round_up_f32(ymid[inside] + kGuard);
      e.lo = round_down_f32(ymid[inside] - kGuard);
      e.tx = t.thr[inside];
      if (!(e.lo > (float)b) || !(e.hi < (float)(b + 1))) return false;
    }
  }
  return true;
}

}  // namespace

const Nf4Tables *host_tables() {
  static Nf4Tables tables;
  static bool ok = false;
  static std::once_flag once;
  std::call_once(once, [] { ok = build(tables); });
  return ok ? &tables : nullptr;
}

}  // namespace ql

// Host-side construction of the 4-bit codebooks and the encoder's bucket tables.
//
// NF4 ([MC] "1. NormalFloat", [TT] §5 "NF4", [GO] "Idea one"): 16 values
// placed at quantiles of a standard normal, normalised to [-1, 1].  Reading
// used here (the pages give no formula): 8 positive quantiles at
// probabilities 1/2 + (d - 1/2) k/8, k = 1..8, 7 negative ones mirrored from
// 1/2 + (d - 1/2) k/7, k = 1..7, plus an exact zero, all divided by the
// quantile at d, where d = (31/32 + 29/30)/2 keeps the outermost quantile
// finite.  The quantiles are evaluated here in long double by bisection on the
// normal CDF written with erfc, then rounded once to float32.
//
// The variants the pages compare NF4 with ([TT] §5, [MC] "What the
// experiments establish"), on the same storage and encoder:
//  INT4: the symmetric absmax integer grid of [TT] §2 at 4 bits, levels q/7
//        for q = -8..7 (q = -8 is never chosen since |x| <= 1);
//  FP4:  the E2M1 values {0, 0.5, 1, 1.5, 2, 3, 4, 6} and their negatives
//        divided by 6, at codes 1..15, with an unused -1.5 at code 0.
// (Readings: the pages fix neither table.)  Each rational is evaluated in
// double and rounded to float32.
//
// Encoder ([TT] §2 "Choose a scale, then round"): the code of a normalised
// value x = fp32(w / absmax) is the number of level midpoints strictly below
// x (nearest level, ties to the lower one).  The GPU evaluates
// y = fma(w, 16 * rcp(absmax), yoff) instead of the division, with
// yoff = 16 + delta; |y - (16x + yoff)| is bounded (see kGuard), so a bucket
// table over floor(y) decides the code except inside a narrow guard band
// around each midpoint, where the kernel falls back to the exact IEEE
// division.  delta (0, 1/2, 1/4 or 3/4, the first that works) keeps every
// midpoint's guard band inside one bucket.

#include <cfloat>
#include <cmath>
#include <mutex>

#include "common.h"

namespace ql {

namespace {

// |y - (16 x + yoff)| <= 16 * 2^-22 (a 2-ulp reciprocal) + 2^-19 (fma rounding, y < 34)
// + 2^-21 (rounding of x itself) = 6.2e-6; use a margin of 1.3x.
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

bool levels_for(int cb, float *lv) {
  if (cb == 0) {
    const long double d = 0.5L * (31.0L / 32.0L + 29.0L / 30.0L);
    const long double top = norm_quantile(d);
    long double v[16];
    int k = 0;
    for (int i = 7; i >= 1; --i) v[k++] = -norm_quantile(0.5L + (d - 0.5L) * i / 7.0L) / top;
    v[k++] = 0.0L;
    for (int i = 1; i <= 8; ++i) v[k++] = norm_quantile(0.5L + (d - 0.5L) * i / 8.0L) / top;
    for (int i = 0; i < 16; ++i) lv[i] = (float)v[i];
    lv[0] = (float)(-norm_quantile(d) / top);  // exactly -1 by construction
    lv[7] = 0.0f;
    return true;
  }
  if (cb == 1) {
    for (int q = -8; q <= 7; ++q) lv[q + 8] = (float)((double)q / 7.0);
    return true;
  }
  if (cb == 2) {
    const double mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    lv[0] = -1.5f;
    for (int i = 0; i < 7; ++i) lv[1 + i] = (float)(-mag[7 - i] / 6.0);
    for (int i = 0; i < 8; ++i) lv[8 + i] = (float)(mag[i] / 6.0);
    return true;
  }
  return false;
}

bool build_buckets(Nf4Tables &t, const double *ymid, double yoff) {
  for (int b = 0; b < kBuckets; ++b) {
    EncBucket &e = t.bucket[b];
    uint32_t below = 0;
    int inside = -1, count = 0;
    for (int j = 0; j < 15; ++j) {
      const double y = ymid[j] + yoff;
      if (y < (double)b) ++below;
      if (y >= (double)b && y < (double)(b + 1)) { inside = j; ++count; }
      // a guard band must never straddle a bucket edge
      if (fabs(y - (double)b) <= kGuard) return false;
    }
    if (count > 1) return false;
    e.base = below;
    if (inside < 0) {
      e.hi = INFINITY;
      e.lo = INFINITY;
      e.tx = INFINITY;
    } else {
      e.hi = round_up_f32(ymid[inside] + yoff + kGuard);
      e.lo = round_down_f32(ymid[inside] + yoff - kGuard);
      e.tx = t.thr[inside];
      if (!(e.lo > (float)b) || !(e.hi < (float)(b + 1))) return false;
    }
  }
  return true;
}

bool build(Nf4Tables &t, int cb) {
  if (!levels_for(cb, t.level)) return false;
  for (int i = 1; i < 16; ++i)
    if (!(t.level[i] > t.level[i - 1])) return false;
  // -1 and +1 are levels (the block's largest magnitude is reproduced exactly); anything
  // below -1 is never chosen
  if (t.level[15] != 1.0f || !(t.level[0] == -1.0f || (t.level[0] < -1.0f && t.level[1] == -1.0f))) return false;
  t.zero_code = 16;
  for (uint32_t i = 0; i < 16; ++i)
    if (t.level[i] == 0.0f) t.zero_code = i;
  if (t.zero_code > 15) return false;

  double ymid[15];
  for (int j = 0; j < 15; ++j) {
    double m = ((double)t.level[j] + (double)t.level[j + 1]) * 0.5;  // exact in double
    t.thr[j] = round_down_f32(m);
    ymid[j] = 16.0 * m;                                                // exact in double
  }
  const double shifts[4] = {0.0, 0.5, 0.25, 0.75};
  for (double d : shifts) {
    if (build_buckets(t, ymid, 16.0 + d)) {
      t.yoff = (float)(16.0 + d);
      return true;
    }
  }
  return false;
}

}  // namespace

const Nf4Tables *host_tables(int codebook) {
  static Nf4Tables tables[kCodebooks];
  static bool ok[kCodebooks];
  static std::once_flag once;
  std::call_once(once, [] {
    for (int c = 0; c < kCodebooks; ++c) ok[c] = build(tables[c], c);
  });
  if (codebook < 0 || codebook >= kCodebooks) return nullptr;
  return ok[codebook] ? &tables[codebook] : nullptr;
}

}  // namespace ql

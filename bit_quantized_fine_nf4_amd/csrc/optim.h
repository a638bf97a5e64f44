// Host-side launcher of the adapter optimizer step.
#pragma once

#include "common.h"

namespace ql {

struct AdamwArgs {
  float *p;
  const float *g;
  float *m;
  float *v;
  uint16_t *pbf;
  int64_t n;
  int64_t step;
  double lr, beta1, beta2, eps, wd;
};
hipError_t launch_adamw(const AdamwArgs &a, hipStream_t st);

}  // namespace ql

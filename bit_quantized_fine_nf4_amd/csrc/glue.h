// Elementwise glue between a transformer block's NF4 linears — host interface.
#pragma once

#include "common.h"

namespace ql {

constexpr int kMaxSumParts = 8;

struct SumParts {
  const uint16_t *p[kMaxSumParts];  // device pointers, the first k used
  int k;
};

hipError_t launch_silu_gate_fwd(const uint16_t *G, const uint16_t *U, int64_t n, uint16_t *H, hipStream_t st);
hipError_t launch_silu_gate_bwd(const uint16_t *G, const uint16_t *U, const uint16_t *dH, int64_t n, uint16_t *dG,
                                uint16_t *dU, hipStream_t st);
hipError_t launch_grad_sum(const SumParts &parts, int64_t n, uint16_t *out, hipStream_t st);

}  // namespace ql

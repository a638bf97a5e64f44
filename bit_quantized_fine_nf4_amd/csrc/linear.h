// Host-side launchers of the NF4 + LoRA linear-layer kernels.
#pragma once

#include "common.h"

namespace ql {

struct LinearArgs {
  const uint8_t *codes;   // [o][h] packed NF4 codes
  const int8_t *qabsmax;  // [o][h/64]
  const float *scale2;    // per 256 block scales
  const float *mean;      // 1 value
  int64_t h, o, M;
  int r;
  float s;
};

// Optional per-thread events recorded around the fused GEMM / GEMV launches
// (0 = forward GEMM, 1 = dX GEMM, 2 = few-token forward).
void set_timing_events(int kernel, hipEvent_t start, hipEvent_t stop);

size_t linear_fwd_workspace(int64_t M, int64_t h, int64_t o, int r);
size_t linear_bwd_workspace(int64_t M, int64_t h, int64_t o, int r);
// false when the adapter gradients of this shape would need more token splits than
// one launch holds (very large M with very wide layers)
bool linear_bwd_supported(int64_t M, int64_t h, int64_t o, int r);
// token splits of the adapter-gradient reduction (each split's operand slab stays
// below 2^31 bytes)
int64_t linear_bwd_token_splits(int64_t M, int64_t h, int64_t o);

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                             uint16_t *Y, uint16_t *T, void *ws, const Nf4Tables &tab, hipStream_t st);
hipError_t launch_linear_bwd(const LinearArgs &a, const uint16_t *X, const uint16_t *T, const uint16_t *dY,
                             const uint16_t *L1, const uint16_t *L2, uint16_t *dX, float *dL1, float *dL2,
                             void *ws, const Nf4Tables &tab, hipStream_t st);

}  // namespace ql

// Host-side launchers of the codec and linear-layer kernels.
#pragma once

#include "common.h"

namespace ql {

hipError_t launch_quantize(const void *w, bool bf16, int64_t n, uint8_t *codes, float *absmax,
                           const Nf4Tables &tab, hipStream_t st);
size_t dq_workspace_bytes();
hipError_t launch_double_quant(const float *absmax, int64_t nb, int8_t *qabsmax, float *scale2,
                               float *mean, void *ws, hipStream_t st);
// The same with the library's own per-device static scratch instead of a workspace
// (hipErrorInvalidDevice when `st` belongs to another device than the current one).
hipError_t launch_double_quant_noalloc(const float *absmax, int64_t nb, int8_t *qabsmax, float *scale2,
                                       float *mean, hipStream_t st);
// absmax != nullptr: no double quantization (qabsmax, scale2, mean unused, may be null).
hipError_t launch_dequantize(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                             const float *mean, int64_t n, void *out, bool bf16, const Nf4Tables &tab,
                             hipStream_t st, const float *absmax = nullptr);

// Adapter merge W' = W_hat + s·L1·L2 ([o][h] storage); mode 0: float32 out,
// 1: bf16 out, 2: NF4 codes_out / absmax_out of W'.
struct MergeArgs {
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t h, o;
  const uint16_t *L1, *L2;
  int r;
  float s;
  void *out;
  uint8_t *codes_out;
  float *absmax_out;
};
hipError_t launch_merge(const MergeArgs &m, int mode, const Nf4Tables &tab, hipStream_t st);

}  // namespace ql

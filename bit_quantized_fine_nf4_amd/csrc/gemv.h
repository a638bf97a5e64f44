// Few-token NF4 forward (M <= 16 tokens) — host interface.
#pragma once

#include "common.h"

namespace ql {

// Y[m][n] = sum_k X[m][k] W_hat[n][k] + sum_q sT[m][q] L2[q][n]  (bf16 out, float32 sums)
//  X [M][ldx] bf16, codes [N][K/2], qabsmax [N][K/64], scale2 per 256 block scales,
//  sT [M][ldt] bf16 with s applied (r > 0), L2 [r][N] bf16, Y [M][ldy] bf16.
//  K and N are multiples of 64, 1 <= M <= 16.
struct GemvParams {
  const uint16_t *X;
  int64_t ldx;
  int M;
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t K, N;
  const uint16_t *sT;
  int ldt;
  int r;
  const uint16_t *L2;
  uint16_t *Y;
  int64_t ldy;
  float level[16];
};

hipError_t launch_nf4_gemv(const GemvParams &p, hipStream_t st);

}  // namespace ql

// Fused NF4 dequant-GEMM (forward and dX directions) — host interface.
#pragma once

#include "common.h"

namespace ql {

// C[M][N] (bf16) = A[M][K]·B[K][N] + A2[M][K2]·B2[K2][N], float32 accumulation.
//  forward (trans = false): A = X [M][h]; B[k][n] = W_hat[n][k], codes row n, K = h, N = o.
//  dX      (trans = true):  A = dY [M][o]; B[k][n] = W_hat[k][n], codes row k, K = o, N = h.
//  LoRA term: A2 = s-scaled rank-r product [M][lda2] (bf16, zero beyond r);
//   forward: B2 = L2 [r][N] (rows >= b2rows read as zero);
//   dX:      B2 = L1 padded to [N][ldb2] (zero beyond r).
struct GemmParams {
  const uint16_t *A;
  int64_t lda;
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t ldw;    // weights per codes row (h)
  int64_t wrows;  // codes rows (o)
  const uint16_t *A2;
  int64_t lda2;
  const uint16_t *B2;
  int64_t ldb2;
  int b2rows;
  int ksteps;   // 64-wide K steps over the dequantized weight
  int ksteps2;  // 64-wide K steps over the LoRA operands
  int64_t M, N;
  uint16_t *C;
  int64_t ldc;
  int tiles_m, tiles_n;
  float level[16];
};

hipError_t launch_nf4_gemm(GemmParams &gp, bool trans, hipStream_t st);
// 256 x bn tiles (bn = 256 or 128) with four waves that decode B in registers, both
// directions (nf4_gemm_wide.hip)
hipError_t launch_nf4_gemm_wide(GemmParams &gp, bool trans, int bn, hipStream_t st);

}  // namespace ql

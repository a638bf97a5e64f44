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

// Output tile (tm, tn) of workgroup `bid`.  The dispatcher deals workgroups to the
// eight XCDs in turn (XCD = bid % 8) and each XCD has its own L2, so each XCD first
// gets a contiguous range of a tile order, and that order walks bands of `band` tile
// rows column by column: 32 tiles on one XCD then cover band x (32 / band) tiles.
// An A tile-row holds 4 (256-wide tiles) or 8 (128-wide) times the bytes of a code
// tile-column, so bands of 4 or 2 rows keep the fewest bytes per XCD; one row (a
// whole row of tiles per XCD) makes every XCD fetch the whole weight (one LLaMA-65B
// block at 2048 tokens: forward and dX GEMMs fetch 641 and 552 MB per launch with one
// row, 385 and 380 MB with four).
__device__ inline void gemm_tile_of(int bid, int tiles_m, int tiles_n, int band, int &tm, int &tn) {
  const int ntiles = tiles_m * tiles_n;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);
  const int b = bid / (band * tiles_n);
  const int rows = tiles_m - b * band < band ? tiles_m - b * band : band;
  const int rr = bid - b * band * tiles_n;
  tn = rr / rows;
  tm = b * band + rr % rows;
}

hipError_t launch_nf4_gemm(GemmParams &gp, bool trans, hipStream_t st);
// 256 x bn tiles (bn = 256 or 128) with four waves that decode B in registers, both
// directions (nf4_gemm_wide.hip)
hipError_t launch_nf4_gemm_wide(GemmParams &gp, bool trans, int bn, hipStream_t st);

}  // namespace ql

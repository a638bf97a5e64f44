// Stream probe for gfx950: the plain HBM streaming rates that the
// bandwidth-bound kernels of this library are measured against.  Not a step of
// the method: a tile reads RD x 1 KB of contiguous source and writes WR x 1 KB
// of contiguous destination (64 lanes x 16 bytes per instruction, fully
// coalesced); each wave takes D tiles per pass, one grid stride apart, issues
// all their loads, then reduces and stores them.  (RD, WR) = (1, 0) is a pure
// read like the GEMV's weight stream; (4, 1) reads four bytes per byte written
// like quantization of bf16 weights; (1, 4) the reverse, like dequantization
// to bf16.  The launch shape (D, workgroups) is an argument so that the caller
// can take the best rate over a sweep as the ceiling.

#include "stream.h"

namespace ql {

template <int RD, int WR, int D>
__global__ __launch_bounds__(256) void stream_probe_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst,
                                                           int64_t ntiles) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  uint32_t acc = 0;
  for (int64_t t0 = wave; t0 < ntiles; t0 += D * nwaves) {
    u32x4 a[D][RD];
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t t = t0 + d * nwaves;
      if (t < ntiles) {
#pragma unroll
        for (int j = 0; j < RD; ++j) a[d][j] = src[(t * RD + j) * 64 + lane];
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t t = t0 + d * nwaves;
      if (t < ntiles) {
        u32x4 x = a[d][0];
#pragma unroll
        for (int j = 1; j < RD; ++j) x ^= a[d][j];
        if constexpr (WR == 0) {
          acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
        } else {
#pragma unroll
          for (int k = 0; k < WR; ++k) dst[(t * WR + k) * 64 + lane] = x + (uint32_t)k;
        }
      }
    }
  }
  if constexpr (WR == 0) {
    // keeps the loads alive; the value is never meant to match
    if (acc == 0x9E3779B9u && lane == 0) dst[0] = u32x4{acc, acc, acc, acc};
  }
}

template <int RD, int WR>
static hipError_t launch_kind(int depth, unsigned grid, const u32x4 *s, u32x4 *d, int64_t ntiles, hipStream_t st) {
  switch (depth) {
    case 1: return launch(stream_probe_kernel<RD, WR, 1>, grid, 256, st, s, d, ntiles);
    case 2: return launch(stream_probe_kernel<RD, WR, 2>, grid, 256, st, s, d, ntiles);
    case 4: return launch(stream_probe_kernel<RD, WR, 4>, grid, 256, st, s, d, ntiles);
    case 8: return launch(stream_probe_kernel<RD, WR, 8>, grid, 256, st, s, d, ntiles);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_probe(int rd, int wr, int depth, int blocks, const void *src, void *dst, int64_t ntiles,
                               hipStream_t st) {
  int64_t grid = blocks;
  if (grid <= 0) grid = (ntiles + 7) / 8 < 8192 ? (ntiles + 7) / 8 : 8192;
  const auto *s = static_cast<const u32x4 *>(src);
  auto *d = static_cast<u32x4 *>(dst);
  if (rd == 1 && wr == 0) return launch_kind<1, 0>(depth, (unsigned)grid, s, d, ntiles, st);
  if (rd == 4 && wr == 1) return launch_kind<4, 1>(depth, (unsigned)grid, s, d, ntiles, st);
  if (rd == 1 && wr == 4) return launch_kind<1, 4>(depth, (unsigned)grid, s, d, ntiles, st);
  return hipErrorInvalidValue;
}

}  // namespace ql

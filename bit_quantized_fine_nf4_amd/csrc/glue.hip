// Elementwise glue between the NF4 linears of a transformer block, for gfx950.
//
// [MC] "A closer look: Design choices and memory costs": adapters sit on every
// linear layer of the block, attention and feed-forward alike.  The feed-forward
// of the LLaMA models the pages name is gated: its gate and up projections G and
// U meet in H = SiLU(G) * U (SiLU(g) = g * sigmoid(g)) before the down
// projection.  Its backward gives dU = dH * SiLU(G) and
// dG = dH * U * sigmoid(G) * (1 + G * (1 - sigmoid(G))).  Where several linears
// read one input (q, k, v, gate and up all read the block input), its gradient
// is the sum of their dX (grad_sum_kernel).
//
// All three are HBM streams: 16-byte loads and stores of eight bf16 values per
// lane, a grid-stride loop over 8-element groups and a scalar tail, float32
// arithmetic, one round-to-nearest-even to bf16 per output.

#include "glue.h"

namespace ql {
namespace {

QL_DEV u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }
// Non-temporal: for inputs this step reads for the last time (the backward's G, U and
// dH, the input-gradient parts; 65B block: SiLU-gate backward 75 -> 71 us, sum 38 ->
// 36 us; the forward, whose G and U the backward reads again, measured 1 us slower)
QL_DEV u32x4 ld16_last(const uint16_t *p) { return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)); }
QL_DEV void st16(uint16_t *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
QL_DEV float bf(uint16_t v) { return __builtin_bit_cast(float, (uint32_t)v << 16); }
QL_DEV uint16_t to_bf16(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

// exp(-g) overflows to +inf for very negative g, which gives sigmoid = 0 as it should.
QL_DEV float sigmoid(float g) { return 1.0f / (1.0f + __expf(-g)); }

QL_DEV float silu_fwd(float g, float u) { return g * sigmoid(g) * u; }
QL_DEV void silu_bwd(float g, float u, float dh, float &dg, float &du) {
  const float s = sigmoid(g);
  du = dh * (g * s);
  dg = dh * u * (s * (1.0f + g * (1.0f - s)));
}

constexpr int kThreads = 256;

inline int grid_for(int64_t groups) {
  int64_t g = (groups + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 16;  // 16 workgroups per compute unit, then the loop strides
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

}  // namespace

__global__ __launch_bounds__(kThreads) void silu_gate_fwd_kernel(const uint16_t *__restrict__ G,
                                                                  const uint16_t *__restrict__ U, int64_t n,
                                                                  uint16_t *__restrict__ H) {
  const int64_t nv = n >> 3, stride = (int64_t)gridDim.x * kThreads;
  const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (int64_t i = first; i < nv; i += stride) {
    const u32x4 g = ld16(G + 8 * i), u = ld16(U + 8 * i);
    u32x4 h;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      h[j] = pack_bf16x2(silu_fwd(bf16_lo(g[j]), bf16_lo(u[j])), silu_fwd(bf16_hi(g[j]), bf16_hi(u[j])));
    st16(H + 8 * i, h);
  }
  for (int64_t i = 8 * nv + first; i < n; i += stride) H[i] = to_bf16(silu_fwd(bf(G[i]), bf(U[i])));
}

__global__ __launch_bounds__(kThreads) void silu_gate_bwd_kernel(const uint16_t *__restrict__ G,
                                                                  const uint16_t *__restrict__ U,
                                                                  const uint16_t *__restrict__ dH, int64_t n,
                                                                  uint16_t *__restrict__ dG,
                                                                  uint16_t *__restrict__ dU) {
  const int64_t nv = n >> 3, stride = (int64_t)gridDim.x * kThreads;
  const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (int64_t i = first; i < nv; i += stride) {
    const u32x4 g = ld16_last(G + 8 * i), u = ld16_last(U + 8 * i), d = ld16_last(dH + 8 * i);
    u32x4 og, ou;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float g0, u0, g1, u1;
      silu_bwd(bf16_lo(g[j]), bf16_lo(u[j]), bf16_lo(d[j]), g0, u0);
      silu_bwd(bf16_hi(g[j]), bf16_hi(u[j]), bf16_hi(d[j]), g1, u1);
      og[j] = pack_bf16x2(g0, g1);
      ou[j] = pack_bf16x2(u0, u1);
    }
    st16(dG + 8 * i, og);
    st16(dU + 8 * i, ou);
  }
  for (int64_t i = 8 * nv + first; i < n; i += stride) {
    float g, u;
    silu_bwd(bf(G[i]), bf(U[i]), bf(dH[i]), g, u);
    dG[i] = to_bf16(g);
    dU[i] = to_bf16(u);
  }
}

// out = sum of the k inputs (in input order, float32), rounded once.  `out` may be
// one of the inputs: every element is read by the thread that writes it.
__global__ __launch_bounds__(kThreads) void grad_sum_kernel(SumParts parts, int64_t n, uint16_t *out) {
  const int64_t nv = n >> 3, stride = (int64_t)gridDim.x * kThreads;
  const int64_t first = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int k = parts.k;
  for (int64_t i = first; i < nv; i += stride) {
    float acc[8];
    {
      const u32x4 v = ld16_last(parts.p[0] + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[2 * j] = bf16_lo(v[j]), acc[2 * j + 1] = bf16_hi(v[j]);
    }
    for (int q = 1; q < k; ++q) {
      const u32x4 v = ld16_last(parts.p[q] + 8 * i);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[2 * j] += bf16_lo(v[j]), acc[2 * j + 1] += bf16_hi(v[j]);
    }
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(acc[2 * j], acc[2 * j + 1]);
    st16(out + 8 * i, o);
  }
  for (int64_t i = 8 * nv + first; i < n; i += stride) {
    float a = bf(parts.p[0][i]);
    for (int q = 1; q < k; ++q) a += bf(parts.p[q][i]);
    out[i] = to_bf16(a);
  }
}

hipError_t launch_silu_gate_fwd(const uint16_t *G, const uint16_t *U, int64_t n, uint16_t *H, hipStream_t st) {
  return launch(silu_gate_fwd_kernel, grid_for((n + 7) / 8), kThreads, st, G, U, n, H);
}

hipError_t launch_silu_gate_bwd(const uint16_t *G, const uint16_t *U, const uint16_t *dH, int64_t n, uint16_t *dG,
                                uint16_t *dU, hipStream_t st) {
  return launch(silu_gate_bwd_kernel, grid_for((n + 7) / 8), kThreads, st, G, U, dH, n, dG, dU);
}

hipError_t launch_grad_sum(const SumParts &parts, int64_t n, uint16_t *out, hipStream_t st) {
  return launch(grad_sum_kernel, grid_for((n + 7) / 8), kThreads, st, parts, n, out);
}

}  // namespace ql

// Adapter optimizer step for gfx950: AdamW on the float32 master copies of L1
// and L2 ([TT] §4 "One QLoRA Training Step, End to End": only the adapters are
// updated; [TT] §7 "Paged Optimizers", [MC] "3. Paged optimizers", [GO] "Idea
// three": optimizer state may live in CPU memory).  The pages do not spell the
// optimizer out; the update is AdamW with decoupled weight decay (Loshchilov
// and Hutter, "Decoupled Weight Decay Regularization"):
//   p <- p * (1 - lr wd);  m <- b1 m + (1 - b1) g;  v <- b2 v + (1 - b2) g^2
//   p <- p - lr / (1 - b1^t) * m / (sqrt(v) / sqrt(1 - b2^t) + eps)
// HBM-bound elementwise stream: 16-byte loads of p, g, m, v (4 elements per
// lane), 16-byte stores of p, m, v and an optional 8-byte bf16 copy of p.
// The state arrays may be device memory or pinned host memory (the paged-state
// analogue: the kernel then streams them over the host link).
// Compiled with -ffp-contract=off: every step rounds separately.

#include "optim.h"

namespace ql {

struct AdamwParams {
  float *p;
  const float *g;
  float *m;
  float *v;
  uint16_t *pbf;  // may be null
  int64_t n;
  float decay;         // 1 - lr * wd
  float beta1, omb1;   // b1, 1 - b1
  float beta2, omb2;   // b2, 1 - b2
  float step_size;     // lr / (1 - b1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - b2^t)
  float eps;
};

QL_DEV void adamw_one(const AdamwParams &a, float &p, float g, float &m, float &v) {
  p = p * a.decay;
  const float m1 = a.beta1 * m, m2 = a.omb1 * g;
  m = m1 + m2;
  const float gg = g * g;
  const float v1 = a.beta2 * v, v2 = a.omb2 * gg;
  v = v1 + v2;
  const float sv = sqrtf(v);
  const float sc = sv * a.inv_sqrt_bc2;
  const float den = sc + a.eps;
  const float q = m / den;
  const float u = a.step_size * q;
  p = p - u;
}

__global__ __launch_bounds__(256) void adamw_kernel(AdamwParams a) {
  const int64_t n4 = a.n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < n4; q += stride) {
    // every value is read and written once per step: non-temporal accesses (the 65B
    // block's 10.0 M adapter parameters: 62-64 -> 55 us)
    f32x4 p = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.p) + q);
    const f32x4 g = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.g) + q);
    f32x4 m = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.m) + q);
    f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.v) + q);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float pe = p[e], me = m[e], ve = v[e];
      adamw_one(a, pe, g[e], me, ve);
      p[e] = pe;
      m[e] = me;
      v[e] = ve;
    }
    __builtin_nontemporal_store(p, reinterpret_cast<f32x4 *>(a.p) + q);
    __builtin_nontemporal_store(m, reinterpret_cast<f32x4 *>(a.m) + q);
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(a.v) + q);
    if (a.pbf) reinterpret_cast<u32x2 *>(a.pbf)[q] = u32x2{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
  }
  // the last n % 4 elements
  if (blockIdx.x == 0 && threadIdx.x < (a.n & 3)) {
    const int64_t e = 4 * n4 + threadIdx.x;
    float p = a.p[e], m = a.m[e], v = a.v[e];
    adamw_one(a, p, a.g[e], m, v);
    a.p[e] = p;
    a.m[e] = m;
    a.v[e] = v;
    if (a.pbf) a.pbf[e] = (uint16_t)(pack_bf16x2(p, 0.0f) & 0xFFFFu);
  }
}

hipError_t launch_adamw(const AdamwArgs &x, hipStream_t st) {
  AdamwParams a{};
  a.p = x.p; a.g = x.g; a.m = x.m; a.v = x.v; a.pbf = x.pbf; a.n = x.n;
  a.decay = (float)(1.0 - x.lr * x.wd);
  a.beta1 = (float)x.beta1;
  a.omb1 = (float)(1.0 - x.beta1);
  a.beta2 = (float)x.beta2;
  a.omb2 = (float)(1.0 - x.beta2);
  a.step_size = (float)(x.lr / (1.0 - pow(x.beta1, (double)x.step)));
  a.inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - pow(x.beta2, (double)x.step)));
  a.eps = (float)x.eps;
  const int64_t n4 = x.n >> 2;
  int64_t grid = (n4 + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 4096 ? 4096 : grid);
  return launch(adamw_kernel, (int)grid, 256, st, a);
}

}  // namespace ql

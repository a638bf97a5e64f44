// NF4 + LoRA linear layer for gfx950: Y = X·W_hat + s·(X·L1)·L2 and its
// backward into dX, dL1, dL2 ([MC] "The algebra", Eq. 3 and Figure 1;
// [TT] §3-§4).  W_hat is never materialised in HBM: every kernel that needs
// it decodes the 4-bit codes in registers, rescales by the double-quantized
// block scale and hands bf16 values to the matrix cores.
//
// Kernels
//   relayout_kernel      tiny bf16 transposes / zero padding of L1, L2
//   skinny_kernel        P = A·Bt^T for a narrow Bt (the rank-r products
//                        X·L1 and dY·L2^T), MFMA 16x16x32, split-K partials
//   skinny_finish        sums the partials, rounds to bf16 (T or U) and
//                        writes the s-scaled copy the GEMM epilogue uses
//   nf4_gemm_kernel      fused dequant-GEMM, MFMA 32x32x16: forward
//                        (B = W_hat, K along h) and dX (B = W_hat^T, K
//                        along o); the rank-r LoRA product is added as extra
//                        K steps on the same accumulators
//   nf4_gemv_kernel      M <= 16 forward: streams the codes once, decodes a
//                        byte (two codes) per LDS lookup, applies the block
//                        scale after each 64-wide MFMA pair
//   lora_grad_kernel     dL1 = s·X^T·U and dL2 = s·T^T·dY: reduction over
//                        tokens, LDS-transposed operands, split over tokens
//   lora_grad_finish     sums the token splits, scales by s, stores dL1
//                        [h][r] or dL2 [r][o]

#include "linear.h"
#include "gemm.h"

namespace ql {

namespace {

inline int64_t rup(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

QL_DEV bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

QL_DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
QL_DEV f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

QL_DEV uint16_t to_bf16(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

}  // namespace

// ---------------------------------------------------------------------------
// dst[a][b] = (a < av && b < bv) ? (trans ? src[b*lds + a] : src[a*lds + b]) : 0
// ---------------------------------------------------------------------------
__global__ void relayout_kernel(const uint16_t *__restrict__ src, int64_t lds, bool trans, int64_t A,
                                int64_t B, int64_t av, int64_t bv, uint16_t *__restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= A * B) return;
  const int64_t a = idx / B, b = idx % B;
  uint16_t v = 0;
  if (a < av && b < bv) v = trans ? src[b * lds + a] : src[a * lds + b];
  dst[idx] = v;
}

// ---------------------------------------------------------------------------
// Rank-r products.  part[s][m][q] = sum over split s of A[m][k] * Bt[q][k].
// A wave owns 16 rows and all NT*16 columns; operands come straight from
// global memory in MFMA fragment order (16 B per lane per K step).
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void skinny_kernel(const uint16_t *__restrict__ A, int64_t lda, int64_t M,
                                                     int64_t K, const uint16_t *__restrict__ Bt, int64_t ldb,
                                                     int rvalid, int64_t kchunk, float *__restrict__ part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t m0 = (int64_t)blockIdx.x * 64 + wave * 16;
  const int64_t kb = (int64_t)blockIdx.y * kchunk;
  const int64_t ke = kb + kchunk < K ? kb + kchunk : K;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t m = m0 + r16;
  const bool mok = m < M;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  const uint16_t *arow = A + (mok ? m : 0) * lda + 8 * g;
#pragma unroll 2
  for (int64_t k = kb; k < ke; k += 32) {
    u32x4 a = mok ? *reinterpret_cast<const u32x4 *>(arow + k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int q = t * 16 + r16;
      u32x4 b = q < rvalid ? *reinterpret_cast<const u32x4 *>(Bt + (int64_t)q * ldb + k + 8 * g)
                           : u32x4{0, 0, 0, 0};
      acc[t] = mfma16(a, b, acc[t]);
    }
  }
  constexpr int RP = NT * 16;
  float *out = part + (int64_t)blockIdx.y * M * RP;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = m0 + 4 * g + v;
      if (row < M) out[row * RP + t * 16 + r16] = acc[t][v];
    }
}

// out1[m][q] = bf16(sum) for q < n1 (row stride ld1; zero for r <= q < n1)
// out2[m][q] = bf16(s * sum) for q < ld2 (zero for q >= r)
__global__ void skinny_finish_kernel(const float *__restrict__ part, int S, int64_t M, int RP, int r, float s,
                                     uint16_t *__restrict__ out1, int ld1, uint16_t *__restrict__ out2, int ld2) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t W = ld2 > ld1 ? ld2 : ld1;
  if (idx >= M * W) return;
  const int64_t m = idx / W;
  const int q = (int)(idx % W);
  float acc = 0.0f;
  if (q < r)
    for (int i = 0; i < S; ++i) acc += part[((int64_t)i * M + m) * RP + q];
  if (out1 && q < ld1) out1[m * ld1 + q] = q < r ? to_bf16(acc) : (uint16_t)0;
  if (out2 && q < ld2) out2[m * ld2 + q] = q < r ? to_bf16(s * acc) : (uint16_t)0;
}

// ---------------------------------------------------------------------------
// Few-token forward (M <= 16): Y = X·W_hat (+ s·T·L2), bandwidth-bound on the
// packed codes.  Matrix-core formulation with the weights as the B operand of
// v_mfma_f32_32x32x16_bf16: lane l owns output row n = n0 + l%32 and lane group
// g = l/32 owns k in [32g, 32g+32) of a 64-block, so one 16-byte code load per
// lane per block feeds four MFMAs (MFMA j takes k = 32g + 8j + 0..7) that span
// exactly one block.  The MFMAs see bf16(level[code]) (a 256-entry LDS table
// maps a code byte to the bf16 pair of its two levels) and the block scale
// a_hat is applied once to the float32 block partial.  Tokens are the MFMA
// rows (rows >= M are zero; only the 16 lowest rows are kept).
// Workgroup: 512 threads = 8 waves over 64 output rows (two 32-row groups that
// share the token fragments); the waves split K and reduce through LDS.
// ---------------------------------------------------------------------------
struct GemvParams {
  const uint16_t *X;
  int64_t ldx;
  int M;
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t K, N;
  const uint16_t *sT;  // [M][ldt] bf16, s already applied (r > 0)
  int ldt;
  int r;
  const uint16_t *L2;  // [r][N] bf16
  uint16_t *Y;
  int64_t ldy;
  float level[16];
};

constexpr int kGemvRows = 64, kGemvWaves = 8, kGemvUnroll = 4;

__global__ __launch_bounds__(512) void nf4_gemv_kernel(GemvParams p) {
  __shared__ uint32_t lut2[256];
  __shared__ float red[kGemvWaves][2][16][33];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 256) lut2[tid] = pack_bf16x2(p.level[tid >> 4], p.level[tid & 15]);
  __syncthreads();

  const int64_t n0 = (int64_t)blockIdx.x * kGemvRows;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t nblk = p.K >> 6;
  const int64_t b0 = wave * nblk / kGemvWaves, b1 = (wave + 1) * nblk / kGemvWaves;
  const float mu = *p.mean;
  const bool mok = l32 < p.M;  // this lane supplies token row l32 of the A operand
  const uint16_t *xrow = p.X + (int64_t)(mok ? l32 : 0) * p.ldx + 32 * g;
  const uint8_t *crow[2];
  const int8_t *qrow[2];
  int64_t blkrow[2];
#pragma unroll
  for (int gr = 0; gr < 2; ++gr) {
    const int64_t n = n0 + 32 * gr + l32;
    crow[gr] = p.codes + n * (p.K >> 1) + 16 * g;
    qrow[gr] = p.qabsmax + n * nblk;
    blkrow[gr] = n * nblk;
  }
  float acc[2][8];
#pragma unroll
  for (int gr = 0; gr < 2; ++gr)
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[gr][v] = 0.0f;

  for (int64_t bb = b0; bb < b1; bb += kGemvUnroll) {
    u32x4 cw[kGemvUnroll][2];
    u32x4 xa[kGemvUnroll][4];
    int8_t qa[kGemvUnroll][2];
    float s2[kGemvUnroll][2];
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int64_t b = bb + u;
      const bool ok = b < b1;
#pragma unroll
      for (int gr = 0; gr < 2; ++gr) {
        cw[u][gr] = ok ? *reinterpret_cast<const u32x4 *>(crow[gr] + b * 32) : u32x4{0x77777777u, 0x77777777u,
                                                                                      0x77777777u, 0x77777777u};
        qa[u][gr] = ok ? qrow[gr][b] : (int8_t)0;
        s2[u][gr] = ok ? p.scale2[(blkrow[gr] + b) >> 8] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xa[u][j] = (ok && mok) ? *reinterpret_cast<const u32x4 *>(xrow + b * 64 + 8 * j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
#pragma unroll
      for (int gr = 0; gr < 2; ++gr) {
        f32x16 t;
#pragma unroll
        for (int v = 0; v < 16; ++v) t[v] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = cw[u][gr][j];
          const u32x4 bw = {lut2[w & 0xFF], lut2[(w >> 8) & 0xFF], lut2[(w >> 16) & 0xFF], lut2[w >> 24]};
          t = mfma32(xa[u][j], bw, t);
        }
        const float ah = scale_hat(qa[u][gr], s2[u][gr], mu);
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[gr][v] = __builtin_fmaf(ah, t[v], acc[gr][v]);
      }
    }
  }
  // acc[gr][v] = partial Y[token i][row n0 + 32gr + l32], i = 8(v/4) + 4g + v%4
#pragma unroll
  for (int gr = 0; gr < 2; ++gr)
#pragma unroll
    for (int v = 0; v < 8; ++v) red[wave][gr][8 * (v >> 2) + 4 * g + (v & 3)][l32] = acc[gr][v];
  __syncthreads();
  // 64 rows x 16 tokens = 1024 outputs, two per thread
  for (int o = tid; o < 2 * 16 * 32; o += 512) {
    const int gr = o / 512, tok = (o / 32) % 16, col = o % 32;
    if (tok >= p.M) continue;
    float y = 0.0f;
#pragma unroll
    for (int w = 0; w < kGemvWaves; ++w) y += red[w][gr][tok][col];
    const int64_t n = n0 + 32 * gr + col;
    for (int q = 0; q < p.r; ++q)
      y = __builtin_fmaf(bf16_lo(p.sT[(int64_t)tok * p.ldt + q]), bf16_lo(p.L2[(int64_t)q * p.N + n]), y);
    p.Y[(int64_t)tok * p.ldy + n] = to_bf16(y);
  }
}

// ---------------------------------------------------------------------------
// Adapter gradients: part[s][i][q] = sum over tokens m of split s of
// P[m][i] * Q[m][q].  Both operands are token-major in HBM; a workgroup
// transposes a 64-token slab of each into LDS ([i][m] and [q][m]) so the
// MFMA fragments are 16-byte LDS reads.  Workgroup = 64 values of i, all q.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(256) void lora_grad_kernel(const uint16_t *__restrict__ P, int64_t ldp, int64_t I,
                                                        const uint16_t *__restrict__ Q, int64_t ldq, int rq,
                                                        int64_t M, int64_t mchunk, float *__restrict__ part) {
  constexpr int RP = NT * 16, LDT = 64 + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Pt[64 * LDT];
  __shared__ __attribute__((aligned(16))) uint16_t Qt[RP * LDT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t i0 = (int64_t)blockIdx.x * 64;
  const int64_t ms = (int64_t)blockIdx.y * mchunk;
  const int64_t me = ms + mchunk < M ? ms + mchunk : M;
  const bool qvec = (ldq % 8) == 0;
  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  for (int64_t mb = ms; mb < me; mb += 64) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int chunk = tid + 256 * c, mm = chunk >> 3, i8 = chunk & 7;
      const int64_t m = mb + mm;
      const u32x4 v = m < me ? *reinterpret_cast<const u32x4 *>(P + m * ldp + i0 + i8 * 8) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 8; ++e) Pt[(i8 * 8 + e) * LDT + mm] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
    }
    for (int chunk = tid; chunk < 64 * (RP / 8); chunk += 256) {
      const int mm = chunk / (RP / 8), q8 = chunk % (RP / 8);
      const int64_t m = mb + mm;
      uint16_t vals[8];
      if (m < me && qvec && q8 * 8 + 8 <= rq) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(Q + m * ldq + q8 * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = (m < me && q8 * 8 + e < rq) ? Q[m * ldq + q8 * 8 + e] : (uint16_t)0;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) Qt[(q8 * 8 + e) * LDT + mm] = vals[e];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const u32x4 af = *reinterpret_cast<const u32x4 *>(Pt + (wave * 16 + (lane & 15)) * LDT + kk * 32 + (lane >> 4) * 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4 bq = *reinterpret_cast<const u32x4 *>(Qt + (t * 16 + (lane & 15)) * LDT + kk * 32 + (lane >> 4) * 8);
        acc[t] = mfma16(af, bq, acc[t]);
      }
    }
    __syncthreads();
  }
  float *out = part + (int64_t)blockIdx.y * I * RP;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t i = i0 + wave * 16 + 4 * (lane >> 4) + v;
      out[i * RP + t * 16 + (lane & 15)] = acc[t][v];
    }
}

// dL[i][q] (trans = false, stride r) or dL[q][i] (trans = true, stride I) = s * sum_s part
__global__ void lora_grad_finish_kernel(const float *__restrict__ part, int S, int64_t I, int RP, int r, float s,
                                        bool trans, float *__restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= I * r) return;
  int64_t i, q;
  if (trans) { q = idx / I; i = idx % I; } else { i = idx / r; q = idx % r; }
  float acc = 0.0f;
  for (int k = 0; k < S; ++k) acc += part[((int64_t)k * I + i) * RP + q];
  out[idx] = s * acc;
}

// ---------------------------------------------------------------------------
// Host side: split choices (shared by workspace sizing and launches), launches.
// ---------------------------------------------------------------------------
namespace {

constexpr int kTargetGroups = 512;

struct Split {
  int S;
  int64_t chunk;
};

Split skinny_split(int64_t M, int64_t K) {
  const int64_t mt = cdiv(M, 64);
  int64_t S = cdiv(kTargetGroups, mt);
  S = S < 1 ? 1 : S;
  S = S > K / 64 ? K / 64 : S;
  int64_t chunk = rup(cdiv(K, S), 64);
  return {(int)cdiv(K, chunk), chunk};
}

Split grad_split(int64_t M, int64_t I) {
  const int64_t it = I / 64;
  int64_t S = cdiv(kTargetGroups, it);
  const int64_t msteps = cdiv(M, 64);
  S = S < 1 ? 1 : S;
  S = S > msteps ? msteps : S;
  int64_t chunk = rup(cdiv(M, S), 64);
  return {(int)cdiv(M, chunk), chunk};
}

struct FwdLayout {
  int RP16, RP64;
  Split sk;
  size_t off_l1t, off_part, off_st, total;
};

FwdLayout fwd_layout(int64_t M, int64_t h, int64_t o, int r) {
  FwdLayout L{};
  if (r == 0) return L;
  L.RP16 = (int)rup(r, 16);
  L.RP64 = (int)rup(r, 64);
  L.sk = skinny_split(M, h);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += rup((int64_t)bytes, 256); return at; };
  L.off_l1t = take((size_t)L.RP16 * h * 2);
  L.off_part = take((size_t)L.sk.S * M * L.RP16 * 4);
  L.off_st = take((size_t)M * L.RP64 * 2);
  L.total = off;
  return L;
}

struct BwdLayout {
  int RP16, RP64;
  Split sk, g1, g2;
  size_t off_part, off_u, off_su, off_l1p, off_g1, off_g2, total;
};

BwdLayout bwd_layout(int64_t M, int64_t h, int64_t o, int r) {
  BwdLayout L{};
  if (r == 0) return L;
  L.RP16 = (int)rup(r, 16);
  L.RP64 = (int)rup(r, 64);
  L.sk = skinny_split(M, o);
  L.g1 = grad_split(M, h);
  L.g2 = grad_split(M, o);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += rup((int64_t)bytes, 256); return at; };
  L.off_part = take((size_t)L.sk.S * M * L.RP16 * 4);
  L.off_u = take((size_t)M * L.RP16 * 2);
  L.off_su = take((size_t)M * L.RP64 * 2);
  L.off_l1p = take((size_t)h * L.RP64 * 2);
  L.off_g1 = take((size_t)L.g1.S * h * L.RP16 * 4);
  L.off_g2 = take((size_t)L.g2.S * o * L.RP16 * 4);
  L.total = off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off); }

void relayout(const uint16_t *src, int64_t lds, bool trans, int64_t A, int64_t B, int64_t av, int64_t bv,
              uint16_t *dst, hipStream_t st) {
  const int64_t n = A * B;
  relayout_kernel<<<(unsigned)cdiv(n, 256), 256, 0, st>>>(src, lds, trans, A, B, av, bv, dst);
}

void skinny(const uint16_t *A, int64_t lda, int64_t M, int64_t K, const uint16_t *Bt, int64_t ldb, int r, int RP16,
            const Split &sp, float *part, hipStream_t st) {
  dim3 grid((unsigned)cdiv(M, 64), (unsigned)sp.S);
  switch (RP16 / 16) {
#define QL_SK(NT) case NT: skinny_kernel<NT><<<grid, 256, 0, st>>>(A, lda, M, K, Bt, ldb, r, sp.chunk, part); break;
    QL_SK(1) QL_SK(2) QL_SK(3) QL_SK(4) QL_SK(5) QL_SK(6) QL_SK(7) QL_SK(8)
#undef QL_SK
  }
}

void lora_grad(const uint16_t *P, int64_t ldp, int64_t I, const uint16_t *Q, int64_t ldq, int r, int RP16,
               int64_t M, const Split &sp, float *part, hipStream_t st) {
  dim3 grid((unsigned)(I / 64), (unsigned)sp.S);
  switch (RP16 / 16) {
#define QL_LG(NT) case NT: lora_grad_kernel<NT><<<grid, 256, 0, st>>>(P, ldp, I, Q, ldq, r, M, sp.chunk, part); break;
    QL_LG(1) QL_LG(2) QL_LG(3) QL_LG(4) QL_LG(5) QL_LG(6) QL_LG(7) QL_LG(8)
#undef QL_LG
  }
}

thread_local hipEvent_t t_ev[3][2] = {};

struct TimedLaunch {
  int k;
  hipStream_t st;
  TimedLaunch(int kernel, hipStream_t s) : k(kernel), st(s) {
    if (t_ev[k][0]) (void)hipEventRecord(t_ev[k][0], st);
  }
  ~TimedLaunch() {
    if (t_ev[k][1]) (void)hipEventRecord(t_ev[k][1], st);
  }
};

void fill_levels(float *dst, const Nf4Tables &tab) {
  for (int i = 0; i < 16; ++i) dst[i] = tab.level[i];
}

}  // namespace

void set_timing_events(int kernel, hipEvent_t start, hipEvent_t stop) {
  t_ev[kernel][0] = start;
  t_ev[kernel][1] = stop;
}

size_t linear_fwd_workspace(int64_t M, int64_t h, int64_t o, int r) { return fwd_layout(M, h, o, r).total; }
size_t linear_bwd_workspace(int64_t M, int64_t h, int64_t o, int r) { return bwd_layout(M, h, o, r).total; }

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                             uint16_t *Y, uint16_t *T, void *ws, const Nf4Tables &tab, hipStream_t st) {
  const FwdLayout L = fwd_layout(a.M, a.h, a.o, a.r);
  uint16_t *sT = nullptr;
  if (a.r > 0) {
    // T = X·L1 (rank r): L1 [h][r] -> L1t [RP16][h]
    uint16_t *L1t = at<uint16_t>(ws, L.off_l1t);
    relayout(L1, a.r, true, L.RP16, a.h, a.r, a.h, L1t, st);
    float *part = at<float>(ws, L.off_part);
    skinny(X, a.h, a.M, a.h, L1t, a.h, a.r, L.RP16, L.sk, part, st);
    sT = at<uint16_t>(ws, L.off_st);
    skinny_finish_kernel<<<(unsigned)cdiv(a.M * (L.RP64 > a.r ? L.RP64 : a.r), 256), 256, 0, st>>>(
        part, L.sk.S, a.M, L.RP16, a.r, a.s, T, a.r, sT, L.RP64);
  }
  if (a.M <= 16) {
    GemvParams gp{};
    gp.X = X; gp.ldx = a.h; gp.M = (int)a.M;
    gp.codes = a.codes; gp.qabsmax = a.qabsmax; gp.scale2 = a.scale2; gp.mean = a.mean;
    gp.K = a.h; gp.N = a.o;
    gp.sT = sT; gp.ldt = L.RP64; gp.r = a.r; gp.L2 = L2;
    gp.Y = Y; gp.ldy = a.o;
    fill_levels(gp.level, tab);
    {
      TimedLaunch tl(2, st);
      nf4_gemv_kernel<<<(unsigned)(a.o / kGemvRows), 512, 0, st>>>(gp);
    }
    return hipGetLastError();
  }
  GemmParams gp{};
  gp.A = X; gp.lda = a.h;
  gp.codes = a.codes; gp.qabsmax = a.qabsmax; gp.scale2 = a.scale2; gp.mean = a.mean;
  gp.ldw = a.h; gp.wrows = a.o;
  gp.A2 = sT; gp.lda2 = L.RP64; gp.B2 = L2; gp.ldb2 = a.o; gp.b2rows = a.r;
  gp.ksteps = (int)(a.h / 64);
  gp.ksteps2 = a.r > 0 ? L.RP64 / 64 : 0;
  gp.M = a.M; gp.N = a.o;
  gp.C = Y; gp.ldc = a.o;
  fill_levels(gp.level, tab);
  {
    TimedLaunch tl(0, st);
    launch_nf4_gemm(gp, false, st);
  }
  return hipGetLastError();
}

hipError_t launch_linear_bwd(const LinearArgs &a, const uint16_t *X, const uint16_t *T, const uint16_t *dY,
                             const uint16_t *L1, const uint16_t *L2, uint16_t *dX, float *dL1, float *dL2,
                             void *ws, const Nf4Tables &tab, hipStream_t st) {
  const BwdLayout L = bwd_layout(a.M, a.h, a.o, a.r);
  uint16_t *sU = nullptr, *L1p = nullptr;
  if (a.r > 0) {
    // U = dY·L2^T: Bt = L2 [r][o] is already k-contiguous
    float *part = at<float>(ws, L.off_part);
    skinny(dY, a.o, a.M, a.o, L2, a.o, a.r, L.RP16, L.sk, part, st);
    uint16_t *U = at<uint16_t>(ws, L.off_u);
    sU = at<uint16_t>(ws, L.off_su);
    skinny_finish_kernel<<<(unsigned)cdiv(a.M * L.RP64, 256), 256, 0, st>>>(part, L.sk.S, a.M, L.RP16, a.r, a.s, U,
                                                                           L.RP16, sU, L.RP64);
    L1p = at<uint16_t>(ws, L.off_l1p);
    relayout(L1, a.r, false, a.h, L.RP64, a.h, a.r, L1p, st);  // L1 [h][r] -> [h][RP64]
    // dL1 = s·X^T·U   (P = X [M][h], Q = U [M][RP16])
    float *g1 = at<float>(ws, L.off_g1);
    lora_grad(X, a.h, a.h, U, L.RP16, a.r, L.RP16, a.M, L.g1, g1, st);
    lora_grad_finish_kernel<<<(unsigned)cdiv(a.h * a.r, 256), 256, 0, st>>>(g1, L.g1.S, a.h, L.RP16, a.r, a.s, false,
                                                                            dL1);
    // dL2 = s·T^T·dY  (P = dY [M][o], Q = T [M][r]); stored [r][o]
    float *g2 = at<float>(ws, L.off_g2);
    lora_grad(dY, a.o, a.o, T, a.r, a.r, L.RP16, a.M, L.g2, g2, st);
    lora_grad_finish_kernel<<<(unsigned)cdiv(a.o * a.r, 256), 256, 0, st>>>(g2, L.g2.S, a.o, L.RP16, a.r, a.s, true,
                                                                            dL2);
  }
  GemmParams gp{};
  gp.A = dY; gp.lda = a.o;
  gp.codes = a.codes; gp.qabsmax = a.qabsmax; gp.scale2 = a.scale2; gp.mean = a.mean;
  gp.ldw = a.h; gp.wrows = a.o;
  gp.A2 = sU; gp.lda2 = L.RP64; gp.B2 = L1p; gp.ldb2 = L.RP64; gp.b2rows = (int)a.h;
  gp.ksteps = (int)(a.o / 64);
  gp.ksteps2 = a.r > 0 ? L.RP64 / 64 : 0;
  gp.M = a.M; gp.N = a.h;
  gp.C = dX; gp.ldc = a.h;
  fill_levels(gp.level, tab);
  {
    TimedLaunch tl(1, st);
    launch_nf4_gemm(gp, true, st);
  }
  return hipGetLastError();
}

}  // namespace ql

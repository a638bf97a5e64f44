// NF4 + LoRA linear layer for gfx950: Y = X·W_hat + s·(X·L1)·L2 and its
// backward into dX, dL1, dL2 ([MC] "The algebra", Eq. 3 and Figure 1;
// [TT] §3-§4).  W_hat is never materialised in HBM: every kernel that needs
// it decodes the 4-bit codes in registers, rescales by the double-quantized
// block scale and hands bf16 values to the matrix cores.
//
// Kernels
//   lora_rank_kernel     the rank-r products T = X·L1 and U = dY·L2^T, split
//                        over K (64-row workgroups, MFMA 16x16x32, factor
//                        chunk staged once in LDS); lora_rank_reduce_kernel
//                        adds the K splits in order and rounds to bf16 with
//                        the s-scaled copy the GEMM's rank-r step uses
//   lora_rank16_kernel   the same products for r <= 16 in one pass: 8- or
//                        16-row workgroups take the whole K, their eight
//                        waves' sums added in LDS (no partials, no reduce)
//   nf4_gemm_kernel      fused dequant-GEMM, MFMA 32x32x16: forward
//                        (B = W_hat, K along h) and dX (B = W_hat^T, K
//                        along o); the rank-r LoRA product is added as extra
//                        K steps on the same accumulators (256x256 tiles
//                        run nf4_gemm_wide_fwd_kernel and
//                        nf4_gemm_wide_dx_kernel instead)
//   (the M <= 16 forward, nf4_gemv1_kernel and nf4_gemv_kernel, is in gemv.hip)
//   nf4_gemv_dx_kernel   M <= 16 dX: streams the codes once in 64-row stages
//                        through LDS; 4-bit transposing reads give each lane
//                        a column's codes, a byte table yields the bf16 MFMA
//                        operand, the block scale rides on dY; one float32
//                        partial per row chunk
//   gemv_dx_finish_kernel  sums the row-chunk partials in order, adds s·U·L1^T
//   lora_grad_kernel     dL1 = s·X^T·U and dL2 = s·T^T·dY in one launch:
//                        reduction over tokens, LDS-transposed operands,
//                        split over tokens; lora_grad_reduce_kernel sums the
//                        splits in order, scales by s and stores dL1 [h][r]
//                        and dL2 [r][o]; both run before the dX GEMM on the
//                        caller's stream (lora_gradp_kernel: r <= 16 in one
//                        pass, 32- or 64-wide tiles over every token)

#include "linear.h"
#include "gemm.h"
#include "gemv.h"

#include <type_traits>


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

typedef short s16x4 __attribute__((ext_vector_type(4)));
// Two transposing LDS reads (ds_read_b64_tr_b16), 4 rows each: in every 16-lane
// group, lane 4j + q names the 8 bytes at row j, columns 4q..4q+3 of a 4 x 16
// bf16 block and lane i receives the block's column i (4 values per read).
QL_DEV u32x4 tr_pair(const uint16_t *lo, const uint16_t *hi) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(hi));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}

// Buffer resource over [base, base + bytes): loads past the end return zero.
QL_DEV __amdgpu_buffer_rsrc_t gv_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

}  // namespace

// ---------------------------------------------------------------------------
// Rank-r products T = X·L1 (forward) and U = dY·L2^T (backward), split over K
// ([MC] "The algebra", Eq. 3: the adapter's down projection; [TT] §4).
// lora_rank_kernel: a workgroup owns 64 rows and one K range (a multiple of 64
// wide); its four waves take 16 rows each and every rank column, with 16x16x32
// MFMAs.  A operand (X or dY, k-contiguous): lane (i, g) loads 16 bytes of row i
// at k + 8g straight into registers, three 64-wide chunks ahead; rows past M read
// as zero.  B operand: L2 [r][o] (backward) is k-contiguous, so its fragments
// are 16-byte loads of L2 rows; L1 [h][r] (forward) is r-contiguous, so each
// 64 x r chunk of it goes into a double-buffered LDS tile with rows padded by
// 16 bytes, and two transposing reads (ds_read_b64_tr_b16) give each lane one
// column's 8 consecutive k.  Each workgroup reads only its own K range of the
// factor, so the factor is read once per 64 rows (the whole factor per
// workgroup made the previous single-pass kernel's factor traffic 8x that of X).
// With one K range the kernel writes the outputs itself; otherwise it stores
// float32 partial sums and lora_rank_reduce_kernel adds them in split order
// (deterministic) and writes them.
// Outputs: out1[m][q] = bf16(sum) (zero for r <= q < ld1) and
// out2[m][q] = bf16(s * sum) (zero for q >= r).  In the backward, the kernel
// that writes the outputs also writes the zero-padded copy L1p [h][ldp] of L1
// that the dX GEMM's rank-r step reads.
// ---------------------------------------------------------------------------
struct RankParams {
  const uint16_t *A;  // [M][lda] bf16
  int64_t lda, M, K;  // K: a multiple of 64
  const uint16_t *B;  // forward: L1 [K][r]; backward: L2 [r][ldb]
  int64_t ldb;
  int r;
  int kper, ks;       // K per split (a multiple of 64) and number of splits
  float *part;        // [ks][M][16 NT] float32 partial sums (ks > 1)
  float s;
  uint16_t *out1;
  int ld1;
  uint16_t *out2;
  int ld2;
  // backward only (L1p == nullptr otherwise)
  const uint16_t *L1;
  int64_t h;
  int ldp;
  uint16_t *L1p;
};

constexpr int kRankRows = 64;  // rows per workgroup: 16 per wave

// The backward's extra duties, spread over a whole grid (gt: this thread's index,
// gn: the grid's thread count).
// Piece idx of L1p in 16-byte units (r a multiple of 8: L1 is 16-byte aligned and
// ldp a multiple of 64, so every piece is whole): L1's or zero.
QL_DEV u32x4 l1p_piece(const RankParams &p, int64_t idx) {
  const int pp = p.ldp >> 3;
  const int64_t a = idx / pp;
  const int b = (int)(idx % pp);
  return b < (p.r >> 3) ? *reinterpret_cast<const u32x4 *>(p.L1 + a * p.r + 8 * b) : u32x4{0, 0, 0, 0};
}
QL_DEV void l1p_store(const RankParams &p, int64_t idx, u32x4 v) {
  const int pp = p.ldp >> 3;
  *reinterpret_cast<u32x4 *>(p.L1p + (idx / pp) * p.ldp + 8 * (idx % pp)) = v;
}

QL_DEV void rank_extras(const RankParams &p, int64_t gt, int64_t gn) {
  if (!p.L1p) return;
  if (p.r % 8 == 0) {
    for (int64_t idx = gt; idx < p.h * (p.ldp >> 3); idx += gn) l1p_store(p, idx, l1p_piece(p, idx));
    return;
  }
  for (int64_t idx = gt; idx < p.h * p.ldp; idx += gn) {
    const int64_t a = idx / p.ldp, b = idx % p.ldp;
    p.L1p[idx] = b < p.r ? p.L1[a * p.r + b] : (uint16_t)0;
  }
}

// KN: the factor is L1 [K][r] (r-contiguous); VEC: r is a multiple of 8, so each
// L1 row starts on a 16-byte boundary and the chunk copies in 16-byte pieces
// (otherwise element by element).  !KN: the factor is L2 [r][ldb] (k-contiguous).
// Either way a chunk of the factor is staged once in LDS for all four waves.
template <int NT, bool KN, bool VEC>
__global__ __launch_bounds__(256) void lora_rank_kernel(RankParams p) {
  constexpr int RP = NT * 16;
  constexpr int LDB = RP + 8;  // KN tile [64 k][LDB]: row stride of the transposing reads
  constexpr int LDK = 64 + 8;  // NK tile [RP q][LDK]: row stride of the 16-byte fragment reads
  constexpr int TILE = KN ? 64 * LDB : RP * LDK;
  constexpr int BV = (8 * RP + 255) / 256;  // 16-byte factor pieces per thread per chunk (at most)
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TILE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int r = p.r;
  const int64_t m0 = (int64_t)blockIdx.x * kRankRows;
  const int64_t mrows = p.M - m0 < kRankRows ? p.M - m0 : kRankRows;
  const int64_t k0 = (int64_t)blockIdx.y * p.kper;
  const int64_t k1 = k0 + p.kper < p.K ? k0 + p.kper : p.K;
  const int nch = (int)((k1 - k0) >> 6);
  const auto rA = gv_rsrc(p.A + m0 * p.lda + k0, mrows * p.lda * 2 - k0 * 2);
  const int voffA = (int)(((16 * wave + i16) * p.lda + 8 * g) * 2);
  // KN: rows [k0, k1) of L1, (k1 - k0) * r contiguous elements;
  // NK: rows [0, r) of L2 from column k0 (rows past r read as zero)
  const auto rB = KN ? gv_rsrc(p.B + k0 * r, (k1 - k0) * r * 2) : gv_rsrc(p.B + k0, (int64_t)r * p.ldb * 2 - k0 * 2);
  int voffB[BV], soffB[BV];
#pragma unroll
  for (int j = 0; j < BV; ++j) {
    const int idx = tid + 256 * j;
    if (KN) {  // piece idx of the chunk's 64 x r contiguous elements
      const int pr = r >> 3;
      voffB[j] = idx < 8 * r ? idx * 16 : (int)0x80000000u;
      soffB[j] = VEC && idx < 8 * r ? (idx / pr) * LDB + (idx % pr) * 8 : 0;
    } else {   // row idx / 8, piece idx % 8 of 64 k
      voffB[j] = idx < 8 * RP ? (int)(((idx >> 3) * p.ldb + (idx & 7) * 8) * 2) : (int)0x80000000u;
      soffB[j] = (idx >> 3) * LDK + (idx & 7) * 8;
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

  struct Chunk {
    u32x4 a[2];
    u32x4 b[BV];
  };
  // a chunk past the split's end is loaded from an offset past every buffer view: the
  // loads return zero without touching memory, and every step issues the same loads
  // (so the compiler's wait counts stay exact)
  constexpr int kPastEnd = 0x7FFF0000;
  auto load = [&](int c, Chunk &C) {
    const bool live = c < nch;
    const int so = __builtin_amdgcn_readfirstlane(live ? c * 128 : kPastEnd);  // bytes of 64 k
    C.a[0] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA, so, 0);
    C.a[1] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA + 64, so, 0);
    if (!KN || VEC) {
      const int sb = KN ? __builtin_amdgcn_readfirstlane(live ? c * 128 * r : kPastEnd) : so;  // KN: 64 rows of r
#pragma unroll
      for (int j = 0; j < BV; ++j) C.b[j] = __builtin_amdgcn_raw_buffer_load_b128(rB, voffB[j], sb, 0);
    }
  };
  // the chunk's factor into LDS buffer `buf`
  auto put = [&](int c, int buf, const Chunk &C) {
    if (!KN || VEC) {
#pragma unroll
      for (int j = 0; j < BV; ++j)
        if (tid + 256 * j < 8 * (KN ? r : RP)) *reinterpret_cast<u32x4 *>(&Bs[buf][soffB[j]]) = C.b[j];
    } else {
      const int sb = __builtin_amdgcn_readfirstlane(c * 128 * r);
      for (int idx = tid; idx < 64 * r; idx += 256) {
        const uint16_t v = __builtin_amdgcn_raw_buffer_load_b16(rB, idx * 2, sb, 0);
        Bs[buf][(idx / r) * LDB + idx % r] = v;
      }
    }
  };
  const int trow = i16 >> 2, tcol = (i16 & 3) * 4;
  auto compute = [&](int buf, const Chunk &C) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        u32x4 b;
        if constexpr (KN) {
          const uint16_t *lo = &Bs[buf][(32 * sub + 8 * g + trow) * LDB + 16 * t + tcol];
          b = tr_pair(lo, lo + 4 * LDB);
        } else {
          b = *reinterpret_cast<const u32x4 *>(&Bs[buf][(16 * t + i16) * LDK + 32 * sub + 8 * g]);
        }
        acc[t] = mfma16(C.a[sub], b, acc[t]);
      }
  };

  // Loads run kDepth chunks ahead in a ring of kDepth + 1 register stages (one
  // chunk ahead left each workgroup waiting a memory latency per chunk).  Chunk c
  // computes from LDS buffer c & 1; chunk c + 1's factor goes to the other buffer
  // after that (whose reads ended at the previous barrier), then one barrier.  The
  // loop runs whole rounds of kRing chunks with no early exit: chunks past the end
  // load as zero and add nothing (the host makes the chunk count a multiple of
  // kRing wherever K allows).
  constexpr int kDepth = 3, kRing = kDepth + 1;
  Chunk C[kRing];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) load(j, C[j]);
  put(0, 0, C[0]);
  __syncthreads();
  for (int c0 = 0; c0 < nch; c0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      const int c = c0 + u;
      load(c + kDepth, C[(u + kDepth) % kRing]);
      __builtin_amdgcn_sched_barrier(0);
      compute(u & 1, C[u]);
      put(c + 1, (u + 1) & 1, C[(u + 1) % kRing]);
      __syncthreads();
    }
  }

  // C layout: lane (q = 16t + i16, g) holds rows 16 wave + 4g + v
  if (p.ks > 1) {
    float *out = p.part + ((int64_t)blockIdx.y * p.M + m0) * RP;
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = 16 * wave + 4 * g + v;
        if (row < mrows) out[(int64_t)row * RP + 16 * t + i16] = acc[t][v];
      }
    return;
  }
  const int W = p.ld1 > p.ld2 ? p.ld1 : p.ld2;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * wave + 4 * g + v, q = 16 * t + i16;
      if (row >= mrows) continue;
      const int64_t m = m0 + row;
      if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = q < r ? to_bf16(acc[t][v]) : (uint16_t)0;
      if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = q < r ? to_bf16(p.s * acc[t][v]) : (uint16_t)0;
    }
  for (int q = RP + i16; q < W; q += 16)  // columns past the rank tiles: zero
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * wave + 4 * g + v;
      if (row >= mrows) continue;
      const int64_t m = m0 + row;
      if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = 0;
      if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = 0;
    }
  rank_extras(p, (int64_t)(blockIdx.y * gridDim.x + blockIdx.x) * 256 + tid, (int64_t)gridDim.x * gridDim.y * 256);
}

// Sum of the K splits' partials in split order, then the outputs (and the
// backward's extras).  One thread per (row, column).
template <int RP>
__global__ __launch_bounds__(256) void lora_rank_reduce_kernel(RankParams p) {
  const int W = p.ld1 > p.ld2 ? p.ld1 : p.ld2;
  const int64_t gt = (int64_t)blockIdx.x * 256 + threadIdx.x, gn = (int64_t)gridDim.x * 256;
  const int64_t stride = p.M * RP;
  for (int64_t idx = gt; idx < p.M * W; idx += gn) {
    const int64_t m = idx / W;
    const int q = (int)(idx % W);
    float sum = 0.0f;
    if (q < p.r) {
      // the partials were written by other workgroups (other L2s): issue eight
      // loads before adding, still in split order
      const float *src = p.part + m * RP + q;
      int k = 0;
      for (; k + 8 <= p.ks; k += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = src[(k + j) * stride];
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += v[j];
      }
      for (; k < p.ks; ++k) sum += src[k * stride];
    }
    if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = q < p.r ? to_bf16(sum) : (uint16_t)0;
    if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = q < p.r ? to_bf16(p.s * sum) : (uint16_t)0;
  }
  rank_extras(p, gt, gn);
}

// ---------------------------------------------------------------------------
// Adapter gradients, both in one launch ([MC] "One training step": only the
// adapters receive gradients; [TT] §4): tiles [0, pa.tiles) compute
// dL1 = s·X^T·U ([h][r]) and the rest dL2 = s·T^T·dY (stored [r][o]).  Each is
// part[split][i][q] = sum over the split's tokens m of P[m][i] * Q[m][q].
// Both operands are token-major in HBM.  A workgroup owns 128 values of i (all
// q) and a token range, walked in 64-token slabs: a slab of P (256-byte row
// runs) and the matching rows of Q (one contiguous run) are copied into LDS as
// they are, with 16-byte stores; the MFMA fragments need 8 consecutive tokens
// per lane, so P's come from transposing LDS reads (ds_read_b64_tr_b16) and
// Q's from transposing reads too when its rows are a multiple of 8 elements
// (2-byte gathers otherwise).  The next two slabs' loads are in flight while
// one is multiplied (two register stages, double-buffered LDS, one barrier per
// slab); loads past the token range read as zero.  With one token split the
// kernel scales by s and stores the tile; otherwise each split stores float32
// partial sums and lora_grad_reduce_kernel adds them in split order
// (deterministic).  The launch boundary orders the two, so no cross-workgroup
// synchronisation is needed (an in-kernel last-arriving reduction paid an
// agent-scope release per workgroup: 58 against 16 us on a 65B projection).
// ---------------------------------------------------------------------------
struct GradProblem {
  const uint16_t *P;  // [M][ldp], the i index runs along a row
  int64_t ldp, I;
  const uint16_t *Q;  // [M][ldq], q < r valid (rows contiguous: ldq elements each)
  int64_t ldq;
  float *out;         // [I][r] (trans = false) or [r][I] (trans = true)
  bool trans;
  int64_t tiles;      // ceil(I / kGradTile)
  int64_t prow;       // first row of this problem in the partial buffer
};

constexpr int kGradTile = 128;  // values of i per workgroup

template <int NT>
__global__ __launch_bounds__(256) void lora_grad_kernel(GradProblem pa, GradProblem pb, int rq, float s, int64_t M,
                                                        int64_t mchunk, int64_t prows, float *__restrict__ part) {
  constexpr int RP = NT * 16;
  constexpr int LP = kGradTile + 8;                   // P slab row stride (elements)
  constexpr int PCH = 64 * kGradTile / 8 / 256;       // 16-byte P chunks per thread per slab
  constexpr int QCH = (64 * RP / 8 + 255) / 256;      // 16-byte Q chunks per thread per slab (at most)
  __shared__ __attribute__((aligned(16))) uint16_t Ps[2][64 * LP];
  // Q slab: rows padded to LQ when ldq is a multiple of 8 (transposing reads), else
  // kept as it is in memory (ldq-element rows, 2-byte gathers)
  constexpr int LQ = RP + 8;
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][64 * LQ];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const bool second = blockIdx.x >= pa.tiles;
  const GradProblem &pr = second ? pb : pa;
  const int64_t tile = second ? blockIdx.x - pa.tiles : blockIdx.x;
  const int64_t i0 = tile * kGradTile;
  const int64_t ms = (int64_t)blockIdx.y * mchunk;
  const int64_t me = ms + mchunk < M ? ms + mchunk : M;
  const int nsteps = (int)((me - ms + 63) / 64);
  const int64_t ldp = pr.ldp, ldq = pr.ldq;
  const bool qtr = (ldq & 7) == 0;  // wave-uniform: one problem per workgroup
  const int qpr = (int)(ldq >> 3);  // 16-byte pieces per Q row (qtr)
  // rows [ms, me) of P from column i0, and of Q; everything past them reads as zero
  const auto rP = gv_rsrc(pr.P + ms * ldp + i0, (me - ms) * ldp * 2 - i0 * 2);
  const auto rQ = gv_rsrc(pr.Q + ms * ldq, (me - ms) * ldq * 2);
  int voffP[PCH], soffP[PCH], voffQ[QCH];
#pragma unroll
  for (int u = 0; u < PCH; ++u) {
    const int ch = tid + 256 * u, row = ch >> 4, col8 = ch & 15;  // 16 chunks per 256-byte row
    voffP[u] = (int)((row * ldp + col8 * 8) * 2);
    soffP[u] = row * LP + col8 * 8;
  }
#pragma unroll
  for (int u = 0; u < QCH; ++u) {
    const int ch = tid + 256 * u;                      // the slab of Q is 128 * ldq contiguous bytes
    voffQ[u] = ch < 8 * ldq ? ch * 16 : (int)0x80000000u;  // past every buffer: reads zero
  }

  f32x4 acc[2][NT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[a][t] = f32x4{0, 0, 0, 0};

  struct Stage {
    u32x4 p[PCH], q[QCH];
  };
  auto load = [&](int st, Stage &S) {
    const int sp = __builtin_amdgcn_readfirstlane((int)(st * 64 * ldp * 2));
    const int sq = __builtin_amdgcn_readfirstlane((int)(st * 128 * ldq));
#pragma unroll
    for (int u = 0; u < PCH; ++u) S.p[u] = __builtin_amdgcn_raw_buffer_load_b128(rP, voffP[u], sp, 0);
#pragma unroll
    for (int u = 0; u < QCH; ++u) S.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rQ, voffQ[u], sq, 0);
  };
  auto put = [&](int buf, const Stage &S) {
#pragma unroll
    for (int u = 0; u < PCH; ++u) *reinterpret_cast<u32x4 *>(&Ps[buf][soffP[u]]) = S.p[u];
#pragma unroll
    for (int u = 0; u < QCH; ++u) {
      const int ch = tid + 256 * u;
      if (ch < 8 * ldq) {
        const int off = qtr ? (ch / qpr) * LQ + (ch % qpr) * 8 : ch * 8;
        *reinterpret_cast<u32x4 *>(&Qs[buf][off]) = S.q[u];
      }
    }
  };
  // lane 4j + qq of a 16-lane group names row k0 + j, columns 4qq..4qq+3 of the transposing read
  const int trow = c16 >> 2, tcol = (c16 & 3) * 4;
  auto compute = [&](int buf) {
#pragma unroll
    for (int mk = 0; mk < 64; mk += 32) {
      u32x4 af[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const uint16_t *lo = &Ps[buf][(mk + 8 * g + trow) * LP + wave * 32 + 16 * a + tcol];
        af[a] = tr_pair(lo, lo + 4 * LP);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int q = 16 * t + c16;
        u32x4 bq;
        if (qtr) {
          // columns past ldq hold stale values; they only reach output columns q >= rq,
          // which are never stored
          const uint16_t *lo = &Qs[buf][(mk + 8 * g + trow) * LQ + 16 * t + tcol];
          bq = tr_pair(lo, lo + 4 * LQ);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {  // unconditional reads inside the slab (ldq <= RP), masked after
            const uint32_t lo = Qs[buf][(mk + 8 * g + 2 * x) * ldq + q];
            const uint32_t hi = Qs[buf][(mk + 8 * g + 2 * x + 1) * ldq + q];
            w[x] = q < rq ? lo | (hi << 16) : 0u;
          }
          bq = u32x4{w[0], w[1], w[2], w[3]};
        }
#pragma unroll
        for (int a = 0; a < 2; ++a) acc[a][t] = mfma16(af[a], bq, acc[a][t]);
      }
    }
  };

  Stage S0, S1;
  load(0, S0);
  __builtin_amdgcn_sched_barrier(0);
  load(1, S1);
  __builtin_amdgcn_sched_barrier(0);
  put(0, S0);
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    load(st + 2, S0);
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    put(1, S1);
    __syncthreads();
    if (st + 1 >= nsteps) break;
    load(st + 3, S1);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    put(0, S0);
    __syncthreads();
  }

  // D layout: lane (q = 16t + c16, g) holds rows i = 4g + v of each 16-row tile
  if (gridDim.y > 1) {
    float *out = part + ((int64_t)blockIdx.y * prows + pr.prow) * RP;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t i = i0 + wave * 32 + 16 * a + 4 * g + v;
          if (i < pr.I) out[i * RP + t * 16 + c16] = acc[a][t][v];
        }
    return;
  }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + wave * 32 + 16 * a + 4 * g + v;
        const int q = t * 16 + c16;
        if (i < pr.I && q < rq) pr.out[pr.trans ? (int64_t)q * pr.I + i : i * rq + q] = s * acc[a][t][v];
      }
}

// Sum of the adapter gradients' token splits, in split order, scaled by s.  A
// workgroup takes 32 rows i of the partial buffer (one problem: h and o are
// multiples of 64) and every rank column; each thread owns RP / 8 outputs and
// issues all their loads of one split before adding them (independent loads, so
// their latencies overlap).  Reads run along q (coalesced); dL2's [r][o] tile is
// transposed through LDS so its stores run along i too.
constexpr int kGradRedRows = 32;

template <int RP>
__global__ __launch_bounds__(256) void lora_grad_reduce_kernel(GradProblem pa, GradProblem pb, int rq, float s,
                                                               int S, int64_t prows, const float *__restrict__ part) {
  constexpr int PER = kGradRedRows * RP / 256;
  __shared__ float tr[RP][kGradRedRows + 1];
  const int tid = threadIdx.x;
  const int64_t row0 = (int64_t)blockIdx.x * kGradRedRows;  // in the partial buffer's row space
  const bool second = row0 >= pa.I;
  const GradProblem &pr = second ? pb : pa;
  const int64_t i0 = row0 - pr.prow;
  const float *base = part + row0 * RP;
  float sum[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) sum[u] = 0.0f;
  // row (tid + 256u) / RP, column % RP; loads of up to 16 / PER splits in flight
  // before they are added in split order
  constexpr int KB = PER >= 16 ? 1 : 16 / PER;
  int k = 0;
  for (; k + KB <= S; k += KB) {
    float v[KB][PER];
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int u = 0; u < PER; ++u) v[j][u] = base[(int64_t)(k + j) * prows * RP + tid + 256 * u];
#pragma unroll
    for (int j = 0; j < KB; ++j)
#pragma unroll
      for (int u = 0; u < PER; ++u) sum[u] += v[j][u];
  }
  for (; k < S; ++k) {
    const float *src = base + (int64_t)k * prows * RP;
    float v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) v[u] = src[tid + 256 * u];
#pragma unroll
    for (int u = 0; u < PER; ++u) sum[u] += v[u];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = tid + 256 * u, il = idx / RP, q = idx % RP;
    if (pr.trans) tr[q][il] = s * sum[u];
    else if (q < rq) pr.out[(i0 + il) * rq + q] = s * sum[u];
  }
  if (!pr.trans) return;
  __syncthreads();
  for (int idx = tid; idx < rq * kGradRedRows; idx += 256) {
    const int q = idx / kGradRedRows, il = idx % kGradRedRows;
    pr.out[(int64_t)q * pr.I + i0 + il] = tr[q][il];
  }
}

// ---------------------------------------------------------------------------
// Ranks up to 16 in one pass ([MC] "The algebra", Eq. 3 and "One training step";
// [TT] §4).  A rank-16 factor is small next to the activations it multiplies, so
// a workgroup can take few rows (or few adapter-gradient columns) and the whole
// reduction: no split partial sums, and no reduce launch, whose fixed cost of a
// few microseconds per launch dominated these products on a 4096-wide
// projection.  Eight waves split the reduction between them, each loading three
// of its 64-wide pieces ahead into registers; the waves' sums are added in wave
// order through LDS (deterministic).  Pieces past the end load from an offset
// past every buffer view, so they read as zero and every wave issues the same
// loads in each round.
// ---------------------------------------------------------------------------
constexpr int kP16Waves = 8;
constexpr int kP16Threads = 64 * kP16Waves;
constexpr int kP16PastEnd = 0x7FFF0000;

// T = X·L1 (KN) or U = dY·L2^T for r <= 16: workgroup = ROWS rows (16, or 8 when
// 16-row workgroups would leave compute units idle; the MFMA rows past them read
// as zero), wave w takes the 64-wide K chunks w, w + 8, ...  The factor's chunk goes
// through the wave's own LDS tile, loaded in whole 128-byte lines: an L1 chunk (64 x
// r elements, 128 r contiguous bytes) into rows padded to 24 elements, read back with
// transposing reads; an L2 chunk (16 rows of 64 k, rows past r reading as zero) into
// rows padded to 72 elements, read back as each lane's 8 consecutive k.  Outputs as
// lora_rank_kernel's.
template <bool KN, bool VEC, int ROWS>
__global__ __launch_bounds__(kP16Threads) void lora_rank16_kernel(RankParams p) {
  constexpr int LDB = 24;  // KN tile [64 k][LDB]
  constexpr int LDK = 72;  // L2 tile [16 q][LDK]
  static_assert(16 * LDK <= 64 * LDB, "both tiles fit the wave's LDS area");
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kP16Waves][64 * LDB];
  __shared__ float red[kP16Waves][16][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int r = p.r;
  const int64_t m0 = (int64_t)blockIdx.x * ROWS;
  const int64_t mrows = p.M - m0 < ROWS ? p.M - m0 : ROWS;
  // backward: the first round of the padded L1 copy's pieces is loaded here and
  // stored after the products, so its latency overlaps them
  const int64_t gt = (int64_t)blockIdx.x * kP16Threads + tid, gn = (int64_t)gridDim.x * kP16Threads;
  const bool l1vec = p.L1p && p.r % 8 == 0;
  const int64_t l1n = l1vec ? p.h * (p.ldp >> 3) : 0;
  const u32x4 l1first = gt < l1n ? l1p_piece(p, gt) : u32x4{0, 0, 0, 0};
  const int kc = (int)(p.K >> 6);
  const int nj = kc > wave ? (kc - wave + kP16Waves - 1) / kP16Waves : 0;
  const auto rA = gv_rsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  const int voffA = (int)((i16 * p.lda + 8 * g) * 2);
  const auto rB = KN ? gv_rsrc(p.B, p.K * r * 2) : gv_rsrc(p.B, (int64_t)r * p.ldb * 2);
  // KN: pieces `lane` and `lane + 64` of the chunk's 8 r pieces; otherwise rows
  // lane / 8 and 8 + lane / 8 of L2, 16-byte piece lane % 8 of the chunk's 64 k
  // (rows past r read as zero)
  const int voffB0 = KN ? (lane < 8 * r ? lane * 16 : (int)0x80000000u)
                        : (int)(((lane >> 3) * p.ldb + (lane & 7) * 8) * 2);
  const int voffB1 = KN ? (lane + 64 < 8 * r ? (lane + 64) * 16 : (int)0x80000000u)
                        : voffB0 + (int)(8 * p.ldb * 2);
  uint16_t *bt = Bs[wave];
  struct Chunk {
    u32x4 a[2], b[2];
  };
  auto load = [&](int j, Chunk &C) {
    const int c = wave + kP16Waves * j;
    const bool live = j < nj;
    const int so = __builtin_amdgcn_readfirstlane(live ? c * 128 : kP16PastEnd);
    C.a[0] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA, so, 0);
    C.a[1] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA + 64, so, 0);
    const int sb = KN ? __builtin_amdgcn_readfirstlane(live ? c * 128 * r : kP16PastEnd) : so;
    C.b[0] = __builtin_amdgcn_raw_buffer_load_b128(rB, voffB0, sb, 0);
    C.b[1] = __builtin_amdgcn_raw_buffer_load_b128(rB, voffB1, sb, 0);
  };
  // the factor's chunk into the wave's tile.  KN: 64 x r elements (columns past r
  // keep stale values; they only reach accumulator columns q >= r, which are never
  // stored); otherwise 16 rows of 64 k.
  auto put = [&](const Chunk &C) {
    if constexpr (!KN) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
        *reinterpret_cast<u32x4 *>(bt + ((lane >> 3) + 8 * h) * LDK + (lane & 7) * 8) = C.b[h];
      return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int pc = lane + 64 * h;
      if (pc >= 8 * r) continue;
      if (VEC) {
        const int pr = r >> 3;
        *reinterpret_cast<u32x4 *>(bt + (pc / pr) * LDB + (pc % pr) * 8) = C.b[h];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int idx = 8 * pc + e;
          bt[(idx / r) * LDB + idx % r] = (uint16_t)(C.b[h][e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  };
  const int trow = i16 >> 2, tcol = (i16 & 3) * 4;
  f32x4 acc = f32x4{0, 0, 0, 0};
  auto compute = [&](const Chunk &C) {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 b;
      if constexpr (KN) {
        const uint16_t *lo = bt + (32 * sub + 8 * g + trow) * LDB + tcol;
        b = tr_pair(lo, lo + 4 * LDB);
      } else {
        b = *reinterpret_cast<const u32x4 *>(bt + i16 * LDK + 32 * sub + 8 * g);
      }
      acc = mfma16(C.a[sub], b, acc);
    }
  };
  // The wave's own LDS tile needs no barrier: a wave's LDS operations complete in
  // order, and the compiler keeps the order of these may-alias accesses.
  constexpr int kDepth = 3, kRing = kDepth + 1;
  Chunk C[kRing];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) load(j, C[j]);
  for (int j0 = 0; j0 < nj; j0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      load(j0 + u + kDepth, C[(u + kDepth) % kRing]);
      put(C[u]);
      compute(C[u]);
    }
  }

  // C layout: lane (q = i16, g) holds rows 4g + v
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wave][4 * g + v][i16] = acc[v];
  __syncthreads();
  if (tid < ROWS * 16) {
    const int row = tid >> 4, q = tid & 15;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kP16Waves; ++w) sum += red[w][row][q];
    if (row < mrows) {
      const int64_t m = m0 + row;
      if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = q < r ? to_bf16(sum) : (uint16_t)0;
      if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = q < r ? to_bf16(p.s * sum) : (uint16_t)0;
    }
  }
  const int W = p.ld1 > p.ld2 ? p.ld1 : p.ld2;
  if (W > 16) {  // the outputs' columns past the rank tile: zero
    const int pad = W - 16;
    for (int idx = tid; idx < ROWS * pad; idx += kP16Threads) {
      const int row = idx / pad, q = 16 + idx % pad;
      if (row >= mrows) continue;
      const int64_t m = m0 + row;
      if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = 0;
      if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = 0;
    }
  }
  if (l1vec) {
    for (int64_t idx = gt; idx < l1n; idx += gn) l1p_store(p, idx, idx == gt ? l1first : l1p_piece(p, idx));
  } else {
    rank_extras(p, gt, gn);
  }
}

// dL1 = s·X^T·U and dL2 = s·T^T·dY in one pass (launched for r <= 16, RP = 16; the
// kernel takes RP up to 64): tiles [0, pa.tiles) are
// dL1's, the rest dL2's, TI values of i by RP (r rounded up to 16) each (pa.tiles,
// pb.tiles count TI-wide tiles here; TI = 32 when 64-wide tiles would leave compute
// units idle).  With a tile count that is a multiple of 8, consecutive tiles go to
// one XCD, whose L2 then serves the neighbours' halves of each 128-byte line.  A
// workgroup takes every token; wave w the 64-token slabs w, w + 8, ...  A slab of P
// (64 rows x 2 TI bytes) and of Q (64 rows of ldq elements, one contiguous run) go
// into the wave's own LDS tiles, P rows padded to TI + 8 elements and Q rows to
// RP + 8, and both come back through transposing reads (8 consecutive tokens per
// lane).  The register ring holds 4, 3 or 2 slabs as RP grows.
template <int TI, int RP>
__global__ __launch_bounds__(kP16Threads) void lora_gradp_kernel(GradProblem pa, GradProblem pb, int rq, float s,
                                                                 int64_t M) {
  constexpr int LP = TI + 8, LQ = RP + 8, PPR = TI / 8;  // P: 16-byte pieces per row
  constexpr int QPL = RP / 8;                            // Q: 16-byte pieces per lane (at most)
  constexpr int NT = TI / 16, NQ = RP / 16;
  constexpr int kTileElems = 64 * LP + 64 * LQ;
  constexpr int kRedFloats = kP16Waves * TI * RP;
  constexpr int kLdsBytes = kP16Waves * kTileElems * 2 > kRedFloats * 4 ? kP16Waves * kTileElems * 2 : kRedFloats * 4;
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  int64_t bid = blockIdx.x;
  const int64_t ntiles = pa.tiles + pb.tiles;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);  // one XCD -> contiguous tiles
  const bool second = bid >= pa.tiles;
  const GradProblem &pr = second ? pb : pa;
  const int64_t tile = second ? bid - pa.tiles : bid;
  const int64_t i0 = tile * TI;
  const int64_t ldp = pr.ldp, ldq = pr.ldq;
  const bool qvec = (ldq & 7) == 0;  // wave-uniform: one problem per workgroup
  const int nslab = (int)((M + 63) / 64);
  const int nj = nslab > wave ? (nslab - wave + kP16Waves - 1) / kP16Waves : 0;
  // rows [0, M) of P from column i0, and of Q; everything past them reads as zero
  const auto rP = gv_rsrc(pr.P + i0, M * ldp * 2 - i0 * 2);
  const auto rQ = gv_rsrc(pr.Q, M * ldq * 2);
  // P piece u of a lane: row lane / PPR + u * 64 / PPR, 16-byte column lane % PPR;
  // Q piece u: bytes 16 (lane + 64 u) of the slab's 128 ldq contiguous bytes (pieces
  // past them read the next slab's rows or zero, and are not stored).  One lane
  // offset each; the pieces differ by scalar offsets.
  constexpr int RPU = 64 / PPR;  // P rows per piece index
  const int voffP = (int)(((lane / PPR) * ldp + (lane % PPR) * 8) * 2);
  const int soffP = (lane / PPR) * LP + (lane % PPR) * 8;
  const int pstep = (int)(RPU * ldp * 2);
  const int voffQ = lane * 16;
  uint16_t *ps = reinterpret_cast<uint16_t *>(lds) + wave * kTileElems;
  uint16_t *qs = ps + 64 * LP;
  struct Slab {
    u32x4 p[PPR], q[QPL];
  };
  auto load = [&](int j, Slab &S) {
    const int sl = wave + kP16Waves * j;
    const bool live = j < nj;
    const int sp = __builtin_amdgcn_readfirstlane(live ? (int)(sl * 64 * ldp * 2) : kP16PastEnd);
    const int sq = __builtin_amdgcn_readfirstlane(live ? (int)(sl * 128 * ldq) : kP16PastEnd);
#pragma unroll
    for (int u = 0; u < PPR; ++u)
      S.p[u] = __builtin_amdgcn_raw_buffer_load_b128(rP, voffP, live ? (int)((unsigned)sp + (unsigned)(u * pstep))
                                                                     : kP16PastEnd, 0);
#pragma unroll
    for (int u = 0; u < QPL; ++u)
      S.q[u] = __builtin_amdgcn_raw_buffer_load_b128(rQ, voffQ, live ? sq + 1024 * u : kP16PastEnd, 0);
  };
  // Q columns past ldq keep stale values; they only reach output columns q >= rq.
  // With ldq not a multiple of 8 (T of a rank that is not), the slab's Q is copied
  // element by element straight from memory instead (its loads not prefetched).
  auto put = [&](int j, const Slab &S) {
#pragma unroll
    for (int u = 0; u < PPR; ++u) *reinterpret_cast<u32x4 *>(ps + soffP + u * RPU * LP) = S.p[u];
    if (qvec) {
      const int pq = (int)(ldq >> 3);
#pragma unroll
      for (int u = 0; u < QPL; ++u) {
        const int pc = lane + 64 * u;
        if (pc < 8 * ldq) *reinterpret_cast<u32x4 *>(qs + (pc / pq) * LQ + (pc % pq) * 8) = S.q[u];
      }
    } else {
      const int lq = (int)ldq;
      const int sl = wave + kP16Waves * j;
      const int sq = __builtin_amdgcn_readfirstlane(j < nj ? (int)(sl * 128 * ldq) : kP16PastEnd);
      for (int idx = lane; idx < 64 * lq; idx += 64)
        qs[(idx / lq) * LQ + idx % lq] = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rQ, idx * 2, sq, 0);
    }
  };
  const int trow = c16 >> 2, tcol = (c16 & 3) * 4;
  f32x4 acc[NT][NQ];
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int t = 0; t < NQ; ++t) acc[a][t] = f32x4{0, 0, 0, 0};
  auto compute = [&]() {
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      u32x4 bq[NQ];
#pragma unroll
      for (int t = 0; t < NQ; ++t) {
        const uint16_t *lq = qs + (32 * sub + 8 * g + trow) * LQ + 16 * t + tcol;
        bq[t] = tr_pair(lq, lq + 4 * LQ);
      }
#pragma unroll
      for (int a = 0; a < NT; ++a) {
        const uint16_t *lp = ps + (32 * sub + 8 * g + trow) * LP + 16 * a + tcol;
        const u32x4 af = tr_pair(lp, lp + 4 * LP);
#pragma unroll
        for (int t = 0; t < NQ; ++t) acc[a][t] = mfma16(af, bq[t], acc[a][t]);
      }
    }
  };
  constexpr int kRing = RP <= 16 ? 4 : (RP <= 32 ? 3 : 2), kDepth = kRing - 1;
  Slab S[kRing];
#pragma unroll
  for (int j = 0; j < kDepth; ++j) load(j, S[j]);
  for (int j0 = 0; j0 < nj; j0 += kRing) {
#pragma unroll
    for (int u = 0; u < kRing; ++u) {
      load(j0 + u + kDepth, S[(u + kDepth) % kRing]);
      put(j0 + u, S[u]);
      compute();
    }
  }

  // D layout: lane (q = 16t + c16, g) holds rows i = 16a + 4g + v; the sums of the
  // eight waves are added in wave order
  __syncthreads();  // every wave is done with its tiles, which the sums overwrite
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int a = 0; a < NT; ++a)
#pragma unroll
    for (int t = 0; t < NQ; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[(wave * TI + 16 * a + 4 * g + v) * RP + 16 * t + c16] = acc[a][t][v];
  __syncthreads();
  for (int idx = tid; idx < TI * RP; idx += kP16Threads) {
    // dL2 ([r][I]) stores run along i, dL1 ([I][r]) stores along q
    const int il = pr.trans ? idx % TI : idx / RP, q = pr.trans ? idx / TI : idx % RP;
    if (q >= rq) continue;
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < kP16Waves; ++w) sum += red[(w * TI + il) * RP + q];
    const int64_t i = i0 + il;
    if (i < pr.I) pr.out[pr.trans ? (int64_t)q * pr.I + i : i * rq + q] = s * sum;
  }
}

// ---------------------------------------------------------------------------
// Host side: split choices (shared by workspace sizing and launches), launches.
// ---------------------------------------------------------------------------
namespace {

// Workgroups the K-split rank-r and token-split gradient launches aim for: one per
// compute unit (the 65B block's seven linears at 2048 tokens, r = 64: rank-r products
// and adapter gradients 4-8 % faster than with 512, 10-30 % slower with 1024; fewer
// splits also mean fewer partial sums to reduce)
constexpr int kTargetGroups = 256;

struct Split {
  int S;
  int64_t chunk;
};

// Largest token chunk whose slab of a token-major operand with rows of `ld` bf16
// values fits one buffer view: the kernel addresses a split's rows with 32-bit
// offsets and its view is capped below 2^31 bytes.
int64_t grad_chunk_cap(int64_t ld) { return ((int64_t)0x7FFFFFF0 / (2 * ld)) / 64 * 64; }

Split grad_split(int64_t M, int64_t I, int64_t maxld) {
  // about kTargetGroups workgroups: more token splits cost more in partial sums than they save
  const int64_t it = cdiv(I, kGradTile);
  int64_t S = cdiv(kTargetGroups, it);
  const int64_t msteps = cdiv(M, 64);
  S = S < 1 ? 1 : S;
  S = S > msteps ? msteps : S;
  int64_t chunk = rup(cdiv(M, S), 64);
  const int64_t cap = grad_chunk_cap(maxld);
  if (chunk > cap) chunk = cap;
  return {(int)cdiv(M, chunk), chunk};
}

// Adapter gradients for r <= 16 in one pass (lora_gradp_kernel) when a slab's 32-bit
// buffer offsets reach every token of the wider operand.  (At r = 64 the one-pass
// kernel measured slower than the split one on the 65B projections, 34 against 25
// us and 63 against 40 us: every workgroup streams the whole 256 KB token-major U or
// T from L2, and its 144 KB of LDS leaves one workgroup per compute unit.)
bool grad_one_pass(int64_t M, int64_t h, int64_t o, int RP16) {
  return RP16 == 16 && M * (h > o ? h : o) * 2 < (int64_t)0x7FFF0000;
}

// K split of a rank-r product over M rows and K (a multiple of 64): about kTargetGroups
// workgroups of 64 rows, each K range a multiple of 64 wide.
struct RankSplit {
  int ks, kper;
};

RankSplit rank_split(int64_t M, int64_t K) {
  const int64_t rb = cdiv(M, kRankRows), kc = K / 64;
  int64_t ks = cdiv(kTargetGroups, rb);
  ks = ks < 1 ? 1 : (ks > kc ? kc : ks);
  // chunks per K range: a multiple of the kernel's four-chunk rounds where K allows
  int64_t per = rup(cdiv(kc, ks), 4);
  per = per > kc ? kc : per;
  return {(int)cdiv(kc, per), (int)(per * 64)};
}

size_t rank_partial_bytes(int64_t M, int64_t K, int RP16) {
  if (RP16 == 16) return 0;  // one pass (lora_rank16_kernel)
  const RankSplit rs = rank_split(M, K);
  return rs.ks > 1 ? (size_t)rs.ks * M * RP16 * 4 : 0;
}

struct FwdLayout {
  int RP16, RP64;
  size_t off_st, off_tp, total;
};

FwdLayout fwd_layout(int64_t M, int64_t h, int64_t o, int r) {
  FwdLayout L{};
  if (r == 0) return L;
  L.RP16 = (int)rup(r, 16);
  L.RP64 = (int)rup(r, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += rup((int64_t)bytes, 256); return at; };
  L.off_st = take((size_t)M * L.RP64 * 2);
  L.off_tp = take(rank_partial_bytes(M, h, L.RP16));
  L.total = off;
  return L;
}

struct BwdLayout {
  int RP16, RP64;
  Split gs;
  int dxc;  // few-token path (M <= 16): row chunks of the dX partial sums
  size_t off_u, off_su, off_l1p, off_g, off_up, off_dxp, total;
};

int gemv_dx_chunks(int64_t h, int64_t o);

BwdLayout bwd_layout(int64_t M, int64_t h, int64_t o, int r) {
  BwdLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += rup((int64_t)bytes, 256); return at; };
  if (M <= 16) {
    L.dxc = gemv_dx_chunks(h, o);
    L.off_dxp = take((size_t)L.dxc * M * h * 4);
  }
  L.total = off;
  if (r == 0) return L;
  L.RP16 = (int)rup(r, 16);
  L.RP64 = (int)rup(r, 64);
  L.gs = grad_split(M, h + o, h > o ? h : o);
  L.off_u = take((size_t)M * L.RP16 * 2);
  L.off_su = take((size_t)M * L.RP64 * 2);
  L.off_l1p = take((size_t)h * L.RP64 * 2);
  L.off_g = take(grad_one_pass(M, h, o, L.RP16) ? 0 : (size_t)L.gs.S * (h + o) * L.RP16 * 4);
  L.off_up = take(rank_partial_bytes(M, o, L.RP16));
  L.total = off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off); }

hipError_t rank_r(RankParams &rp, bool kn, int RP16, float *part, hipStream_t st) {
  if (RP16 == 16) {
    // 8-row workgroups while 16-row ones would number fewer than the compute units
    if (cdiv(rp.M, 16) < 256) {
      const unsigned grid = (unsigned)cdiv(rp.M, 8);
      if (!kn) return launch(lora_rank16_kernel<false, true, 8>, grid, kP16Threads, st, rp);
      return rp.r % 8 == 0 ? launch(lora_rank16_kernel<true, true, 8>, grid, kP16Threads, st, rp)
                           : launch(lora_rank16_kernel<true, false, 8>, grid, kP16Threads, st, rp);
    }
    const unsigned grid = (unsigned)cdiv(rp.M, 16);
    if (!kn) return launch(lora_rank16_kernel<false, true, 16>, grid, kP16Threads, st, rp);
    return rp.r % 8 == 0 ? launch(lora_rank16_kernel<true, true, 16>, grid, kP16Threads, st, rp)
                         : launch(lora_rank16_kernel<true, false, 16>, grid, kP16Threads, st, rp);
  }
  const RankSplit rs = rank_split(rp.M, rp.K);
  rp.ks = rs.ks;
  rp.kper = rs.kper;
  rp.part = part;
  const dim3 grid((unsigned)cdiv(rp.M, kRankRows), (unsigned)rs.ks);
  const bool vec = rp.r % 8 == 0;
  hipError_t e = hipErrorInvalidValue;
  switch (RP16 / 16) {
#define QL_RK(NT)                                                                              \
  case NT:                                                                                     \
    e = !kn ? launch(lora_rank_kernel<NT, false, true>, grid, 256, st, rp)                     \
            : (vec ? launch(lora_rank_kernel<NT, true, true>, grid, 256, st, rp)               \
                   : launch(lora_rank_kernel<NT, true, false>, grid, 256, st, rp));           \
    if (e == hipSuccess && rs.ks > 1) {                                                        \
      int64_t rg = cdiv(rp.M * (rp.ld1 > rp.ld2 ? rp.ld1 : rp.ld2), 256);                      \
      rg = rg > 2048 ? 2048 : rg;                                                              \
      e = launch(lora_rank_reduce_kernel<NT * 16>, (unsigned)rg, 256, st, rp);                 \
    }                                                                                          \
    break;
    QL_RK(1) QL_RK(2) QL_RK(3) QL_RK(4) QL_RK(5) QL_RK(6) QL_RK(7) QL_RK(8)
#undef QL_RK
  }
  return e;
}

hipError_t lora_grad(const GradProblem &pa, const GradProblem &pb, int r, float s, int64_t M, int RP16,
                     const Split &sp, float *part, hipStream_t st) {
  if (grad_one_pass(M, pa.I, pb.I, RP16)) {
    // 32-wide tiles while 64-wide ones would number fewer than the compute units
    const bool narrow = cdiv(pa.I, 64) + cdiv(pb.I, 64) < 256;
    GradProblem a = pa, b = pb;
    a.tiles = cdiv(a.I, narrow ? 32 : 64);
    b.tiles = cdiv(b.I, narrow ? 32 : 64);
    const unsigned grid = (unsigned)(a.tiles + b.tiles);
    return narrow ? launch(lora_gradp_kernel<32, 16>, grid, kP16Threads, st, a, b, r, s, M)
                  : launch(lora_gradp_kernel<64, 16>, grid, kP16Threads, st, a, b, r, s, M);
  }
  dim3 grid((unsigned)(pa.tiles + pb.tiles), (unsigned)sp.S);
  const int64_t prows = pa.I + pb.I;
  const unsigned rgrid = (unsigned)(prows / kGradRedRows);
  hipError_t e = hipErrorInvalidValue;
  switch (RP16 / 16) {
#define QL_LG(NT)                                                                                   \
  case NT:                                                                                          \
    e = launch(lora_grad_kernel<NT>, grid, 256, st, pa, pb, r, s, M, sp.chunk, prows, part);        \
    if (e == hipSuccess && sp.S > 1)                                                                \
      e = launch(lora_grad_reduce_kernel<NT * 16>, rgrid, 256, st, pa, pb, r, s, sp.S, prows,       \
                 (const float *)part);                                                              \
    break;
    QL_LG(1) QL_LG(2) QL_LG(3) QL_LG(4) QL_LG(5) QL_LG(6) QL_LG(7) QL_LG(8)
#undef QL_LG
  }
  return e;
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

// ---------------------------------------------------------------------------
// Few-token backward: dX = dY·Ŵᵀ + s·U·L1ᵀ for M <= 16 ([MC] "One training
// step": gradients flow through the frozen dequantized weight; [TT] §4).
// HBM-bound like the forward GEMV, but the sum runs down the columns of the
// stored [o][h] weight.  A workgroup takes 512 columns and a chunk of rows and
// writes one float32 partial per (token, column); the finish kernel sums the row
// chunks in order (deterministic), adds s·U·L1ᵀ and rounds to bf16.
// ---------------------------------------------------------------------------
struct GvdParams {
  const uint16_t *dY;  // [M][ldy] bf16
  int64_t ldy;
  int M;
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t h, o;  // W is [o][h]
  int rows;      // rows per chunk (a multiple of kGvmRows)
  float *part;   // [chunks][M][h]
  float level[16];
};

constexpr int kGvdCols = 512;  // columns per workgroup
constexpr int kGvmRows = 64;   // rows (of o) per stage

int gemv_dx_chunks(int64_t h, int64_t o) {
  // about 512 workgroups (two per compute unit), whole stages per chunk
  const int64_t ct = (h + kGvdCols - 1) / kGvdCols;
  const int64_t target = 512;
  int64_t rc = (target + ct - 1) / ct;
  // a chunk's codes stay under 2^30 bytes (32-bit buffer offsets)
  const int64_t minc = (o * (h >> 1) + (int64_t(1) << 30) - 1) >> 30;
  rc = rc > minc ? rc : minc;
  const int64_t maxc = o / 64 > 0 ? o / 64 : 1;
  rc = rc < 1 ? 1 : (rc > maxc ? maxc : rc);
  const int64_t rows = rup((o + rc - 1) / rc, kGvmRows);
  return (int)((o + rows - 1) / rows);
}

// The few-token dX kernel runs on the matrix cores: 16x16x32 bf16 MFMAs take the
// tokens as their rows (padded to 16; on an 8192 x 28672 weight 1, 4 and 16
// tokens take 35, 38 and 44 us, where a v_dot2 kernel took 42, 55 and 114).  A
// workgroup of 8 waves takes 512 columns, wave w the 64-column block w; a stage
// is 64 rows of o.
//   - The stage's raw codes (64 rows x 256 bytes) go to LDS by direct-to-LDS
//     loads, kGvmBufs - 1 stages ahead, in 16-byte chunks placed at
//     chunk ^ (row % 16) within their row.
//   - B: one 4-bit transposing LDS read (ds_read_b64_tr_b4) gives lane i of a
//     16-lane group g the codes of rows 16 g .. 16 g + 15 of one column; each code
//     byte (two consecutive rows) indexes a table of bf16 level pairs, which is
//     exactly an MFMA B dword.  The low 8 rows feed one MFMA, the high 8 another.
//   - A: the block scale rides here: bf16(dY[token][n] * a_hat[n][block]) for the
//     same rows n (tokens past M read as zero).  Each stage's 512 a_hat values are
//     published in LDS by the 512 threads, one each.
// The 4-bit read returns a byte's low nibble first, so lane i of a group holds
// column i ^ 1 (the stored byte keeps the even column in its high nibble).
// Columns past h decode whatever the buffer holds (finite levels) and are never
// stored.  Chunks hold whole stages.
constexpr int kGvmThreads = 512;             // 8 waves: one 64-column block each
constexpr int kGvmRowB = kGvdCols / 2;       // code bytes of a stage row
constexpr int kGvmBufs = 2;                  // code stages held in LDS (3, with 16 table copies: 5-10 % slower)
constexpr int kGvmLutCopies = 32;            // interleaved copies of the byte table (fewer bank conflicts)
static_assert(kGvmThreads == kGvdCols && kGvmThreads == 8 * kGvmRows, "one wave per block, one a_hat per thread");
static_assert(kGvmRows * kGvmRowB == 2 * 16 * kGvmThreads, "two 16-byte loads per thread and stage");

QL_DEV void lds_load16(__amdgpu_buffer_rsrc_t r, void *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
QL_DEV u32x2 tr4(const uint8_t *p) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(p)));
}

struct GvmRegs {
  u32x4 a0, a1;  // dY[token][rows 16 g .. 16 g + 7] and [16 g + 8 .. 16 g + 15] of the stage (bf16)
  uint32_t q;    // int8 block scale of this thread's (row, block), zero-extended
  float s2;      // its second-level scale
};

__global__ __launch_bounds__(kGvmThreads) void nf4_gemv_dx_kernel(GvdParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t cb[kGvmBufs][kGvmRows * kGvmRowB];
  // lut[kGvmLutCopies * byte + copy] = bf16 pair (level[low nibble], level[high nibble])
  __shared__ uint32_t lut[256 * kGvmLutCopies];
  __shared__ __attribute__((aligned(16))) float ahs[2][kGvdCols / 64][kGvmRows];  // a_hat per [block][row]
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < 256 * kGvmLutCopies; i += kGvmThreads) {
    const int e = i / kGvmLutCopies;
    lut[i] = pack_bf16x2(p.level[e & 15], p.level[e >> 4]);
  }
  const int64_t h = p.h, nblk = h >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kGvdCols;
  const int64_t n0 = (int64_t)blockIdx.y * p.rows;
  const int64_t n1 = n0 + p.rows < p.o ? n0 + p.rows : p.o;
  const int nst = (int)((n1 - n0) / kGvmRows);
  const float mu = *p.mean;
  // rows past n1 read as zero codes and scales (and meet no stage)
  const auto rc = gv_rsrc(p.codes + n0 * (h >> 1), (n1 - n0) * (h >> 1));
  const auto rq = gv_rsrc(p.qabsmax + n0 * nblk, (n1 - n0) * nblk);
  const auto rs = gv_rsrc(p.scale2, ((p.o * nblk + kChunk - 1) / kChunk) * 4);
  const auto ry = gv_rsrc(p.dY, (int64_t)p.M * p.ldy * 2);
  const int rowB = (int)(h >> 1);
  // code loads: wave w's load j fills the stage's LDS bytes [1024 (2w + j), +1024),
  // rows 4 (2w + j) .. + 3; lane L takes row r = 4 (2w + j) + L / 16 and puts its
  // logical chunk (L % 16) ^ (r % 16) at physical chunk L % 16
  int vcode[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 4 * (2 * wave + j) + (lane >> 4);
    vcode[j] = r * rowB + (int)(c0 >> 1) + 16 * ((lane & 15) ^ (r & 15));
  }
  // scale role: thread t publishes a_hat of stage row t / 8, block t % 8
  const int srow = tid >> 3, sblk = tid & 7;
  const int voq = (int)(srow * nblk + (c0 >> 6) + sblk);
  const int64_t blk0 = (n0 + srow) * nblk + (c0 >> 6) + sblk;
  // MFMA role: lane (i = lane % 16, g = lane / 16)
  const int i16 = lane & 15, g = lane >> 4;
  const int voy = (int)((i16 * p.ldy + n0 + 16 * g) * 2);  // tokens >= M: past the buffer, zero
  const int lcopy = lane % kGvmLutCopies;

  auto load_codes = [&](int st_) {
    const int st = __builtin_amdgcn_readfirstlane(st_);
    uint8_t *base = &cb[st % kGvmBufs][0];
#pragma unroll
    for (int j = 0; j < 2; ++j) lds_load16(rc, base + 1024 * (2 * wave + j), vcode[j], st * kGvmRows * rowB);
  };
  auto load_regs = [&](int st_, GvmRegs &R) {
    const int st = __builtin_amdgcn_readfirstlane(st_);
    R.a0 = __builtin_amdgcn_raw_buffer_load_b128(ry, voy, st * kGvmRows * 2, 0);
    R.a1 = __builtin_amdgcn_raw_buffer_load_b128(ry, voy + 16, st * kGvmRows * 2, 0);
    R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, voq, st * kGvmRows * (int)nblk, 0);
    R.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                         rs, (int)(((blk0 + (int64_t)st * kGvmRows * nblk) >> 8) * 4), 0, 0));
  };
  auto put = [&](const GvmRegs &R, int buf) {
    ahs[buf][sblk][srow] = scale_hat((int8_t)(R.q & 0xFF), R.s2, mu);
  };
  // vmcnt wait (the direct-to-LDS loads are invisible to the compiler's own waits)
  auto wait_vm = [](auto nconst) {
    constexpr int n = decltype(nconst)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  };
  // loads issued after a stage's code loads and before its wait: that stage's
  // register loads (4) and, with three buffers, the next stage's code loads (2)
  // and register loads (4)
  constexpr int kAfter = kGvmBufs == 3 ? 10 : 4;
  static_assert(kGvmBufs == 2 || kGvmBufs == 3, "two or three code buffers");

  f32x4 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) acc[t] = f32x4{0, 0, 0, 0};
  auto compute = [&](int st, const u32x4 &a0, const u32x4 &a1) {
    const float *sp = &ahs[st & 1][wave][16 * g];
    const f32x4 s0 = *reinterpret_cast<const f32x4 *>(sp), s1 = *reinterpret_cast<const f32x4 *>(sp + 4);
    const f32x4 s2 = *reinterpret_cast<const f32x4 *>(sp + 8), s3 = *reinterpret_cast<const f32x4 *>(sp + 12);
    const u32x4 A0{pack_bf16x2(bf16_lo(a0[0]) * s0[0], bf16_hi(a0[0]) * s0[1]),
                   pack_bf16x2(bf16_lo(a0[1]) * s0[2], bf16_hi(a0[1]) * s0[3]),
                   pack_bf16x2(bf16_lo(a0[2]) * s1[0], bf16_hi(a0[2]) * s1[1]),
                   pack_bf16x2(bf16_lo(a0[3]) * s1[2], bf16_hi(a0[3]) * s1[3])};
    const u32x4 A1{pack_bf16x2(bf16_lo(a1[0]) * s2[0], bf16_hi(a1[0]) * s2[1]),
                   pack_bf16x2(bf16_lo(a1[1]) * s2[2], bf16_hi(a1[1]) * s2[3]),
                   pack_bf16x2(bf16_lo(a1[2]) * s3[0], bf16_hi(a1[2]) * s3[1]),
                   pack_bf16x2(bf16_lo(a1[3]) * s3[2], bf16_hi(a1[3]) * s3[3])};
    // lane i of group g names row 16 g + i; the block's bytes 32 w + 8 t .. + 7 are
    // logical chunk 2 w + t / 2, half t % 2
    const uint8_t *rowp = &cb[st % kGvmBufs][(16 * g + i16) * kGvmRowB];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const u32x2 v = tr4(rowp + 16 * ((2 * wave + (t >> 1)) ^ i16) + 8 * (t & 1));
      u32x4 b0, b1;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        b0[d] = lut[((v[0] >> (8 * d)) & 0xFF) * kGvmLutCopies + lcopy];
        b1[d] = lut[((v[1] >> (8 * d)) & 0xFF) * kGvmLutCopies + lcopy];
      }
      acc[t] = mfma16(A0, b0, acc[t]);
      acc[t] = mfma16(A1, b1, acc[t]);
    }
  };
  auto step = [&](int st, GvmRegs &Rcur, GvmRegs &Rnext) {
    // Rcur: stage st (dY fragments needed now), refilled with stage st + 2;
    // Rnext: stage st + 1 (its a_hat is published here)
    const u32x4 a0 = Rcur.a0, a1 = Rcur.a1;
    __builtin_amdgcn_sched_barrier(0);
    load_codes(st + kGvmBufs - 1);
    __builtin_amdgcn_sched_barrier(0);  // the waits count loads in this order
    load_regs(st + 2, Rcur);
    __builtin_amdgcn_sched_barrier(0);
    compute(st, a0, a1);
    put(Rnext, (st + 1) & 1);
    wait_vm(std::integral_constant<int, kAfter>{});  // stage st + 1's codes in LDS
    __syncthreads();
  };
  GvmRegs R0, R1;
  load_codes(0);
  __builtin_amdgcn_sched_barrier(0);
  load_regs(0, R0);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kGvmBufs == 3) load_codes(1);
  __builtin_amdgcn_sched_barrier(0);
  load_regs(1, R1);
  __builtin_amdgcn_sched_barrier(0);
  put(R0, 0);
  wait_vm(std::integral_constant<int, kAfter>{});  // stage 0's codes in LDS
  __syncthreads();                                 // and the table, and stage 0's a_hat
  int st = 0;
  for (; st + 1 < nst; st += 2) {
    step(st, R0, R1);
    step(st + 1, R1, R0);
  }
  if (st < nst) compute(st, R0.a0, R0.a1);
  wait_vm(std::integral_constant<int, 0>{});  // no load outlives the workgroup

  // D layout: lane (n = lane % 16, g) holds tokens 4g + v of column 64 wave + 16 t + (n ^ 1)
  float *outp = p.part + (int64_t)blockIdx.y * p.M * h;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int64_t col = c0 + 64 * wave + 16 * t + (i16 ^ 1);
    if (col >= h) continue;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * g + v;
      if (m < p.M) outp[(int64_t)m * h + col] = acc[t][v];
    }
  }
}

// dX[m][k..k+7] = bf16(sum of the row-chunk partials + s·U[m]·L1[k..k+7]ᵀ); sU is the
// s-scaled bf16 U ([M][ldsu]), L1 [h][r] bf16.  Block b takes token b / cg and 64
// groups of 8 columns; wave w sums the chunks c = w, w + 4, ... and the four waves
// meet in LDS in a fixed order.
__global__ __launch_bounds__(256) void gemv_dx_finish_kernel(const float *part, int chunks, int M, int64_t h,
                                                             const uint16_t *sU, int ldsu, const uint16_t *L1,
                                                             int r, uint16_t *dX, int64_t ldx) {
  __shared__ float red[4][64][9];
  const int64_t groups = h / 8;
  const int64_t cg = (groups + 63) / 64;
  const int m = (int)(blockIdx.x / cg);
  const int64_t grp = 64 * (int64_t)(blockIdx.x % cg) + (threadIdx.x & 63);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const bool live = grp < groups;
  const int64_t k = (live ? grp : groups - 1) * 8;
  float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  // wave w adds chunks w, w + 4, ... in order, four chunks' loads in flight at a time
  auto add = [&](const f32x4 &a, const f32x4 &b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[i];
      v[4 + i] += b[i];
    }
  };
  int c = w;
  for (; c + 12 < chunks; c += 16) {
    f32x4 a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float *src = part + ((int64_t)(c + 4 * j) * M + m) * h + k;
      a[j] = *reinterpret_cast<const f32x4 *>(src);
      b[j] = *reinterpret_cast<const f32x4 *>(src + 4);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) add(a[j], b[j]);
  }
  for (; c < chunks; c += 4) {
    const float *src = part + ((int64_t)c * M + m) * h + k;
    add(*reinterpret_cast<const f32x4 *>(src), *reinterpret_cast<const f32x4 *>(src + 4));
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[w][l][i] = v[i];
  __syncthreads();
  if (w != 0 || !live) return;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (red[0][l][i] + red[1][l][i]) + (red[2][l][i] + red[3][l][i]);
  if (r > 0) {
    float t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int q = 0; q < r; ++q) {
      const float su = bf16_lo(sU[(int64_t)m * ldsu + q]);
#pragma unroll
      for (int i = 0; i < 8; ++i) t[i] += su * bf16_lo(L1[(k + i) * r + q]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] += t[i];
  }
  *reinterpret_cast<u32x4 *>(dX + (int64_t)m * ldx + k) =
      u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

void fill_levels(float *dst, const Nf4Tables &tab) {
  for (int i = 0; i < 16; ++i) dst[i] = tab.level[i];
}

// The few-token kernel addresses a workgroup's 64 code rows, a row's block scales
// and a token's activations with 32-bit offsets; larger shapes take the GEMM.
bool gemv_fits(const LinearArgs &a) {
  const int64_t lim = (int64_t)1 << 30;
  return 64 * (a.h / 2) < lim && a.o * (a.h / 64) < lim && 16 * a.h * 2 < lim;
}

}  // namespace

void set_timing_events(int kernel, hipEvent_t start, hipEvent_t stop) {
  t_ev[kernel][0] = start;
  t_ev[kernel][1] = stop;
}

size_t linear_fwd_workspace(int64_t M, int64_t h, int64_t o, int r) { return fwd_layout(M, h, o, r).total; }
size_t linear_bwd_workspace(int64_t M, int64_t h, int64_t o, int r) { return bwd_layout(M, h, o, r).total; }

bool linear_bwd_supported(int64_t M, int64_t h, int64_t o, int r) {
  // the adapter-gradient launch has one grid row per token split
  return r == 0 || grad_one_pass(M, h, o, (int)rup(r, 16)) || grad_split(M, h + o, h > o ? h : o).S <= 65535;
}

int64_t linear_bwd_token_splits(int64_t M, int64_t h, int64_t o) {
  return grad_split(M, h + o, h > o ? h : o).S;
}

hipError_t launch_linear_fwd(const LinearArgs &a, const uint16_t *X, const uint16_t *L1, const uint16_t *L2,
                             uint16_t *Y, uint16_t *T, void *ws, const Nf4Tables &tab, hipStream_t st) {
  const FwdLayout L = fwd_layout(a.M, a.h, a.o, a.r);
  uint16_t *sT = nullptr;
  if (a.r > 0) {
    // T = X·L1 (rank r) and its s-scaled, zero-padded copy sT for the GEMM's rank-r step
    sT = at<uint16_t>(ws, L.off_st);
    RankParams rp{};
    rp.A = X; rp.lda = a.h; rp.M = a.M; rp.K = a.h;
    rp.B = L1; rp.ldb = a.r; rp.r = a.r; rp.s = a.s;
    rp.out1 = T; rp.ld1 = a.r; rp.out2 = sT; rp.ld2 = L.RP64;
    const hipError_t e = rank_r(rp, true, L.RP16, at<float>(ws, L.off_tp), st);
    if (e != hipSuccess) return e;
  }
  if (a.M <= 16 && gemv_fits(a)) {
    GemvParams gp{};
    gp.X = X; gp.ldx = a.h; gp.M = (int)a.M;
    gp.codes = a.codes; gp.qabsmax = a.qabsmax; gp.scale2 = a.scale2; gp.mean = a.mean;
    gp.K = a.h; gp.N = a.o;
    gp.sT = sT; gp.ldt = L.RP64; gp.r = a.r; gp.L2 = L2;
    gp.Y = Y; gp.ldy = a.o;
    fill_levels(gp.level, tab);
    TimedLaunch tl(2, st);
    return launch_nf4_gemv(gp, st);
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
  TimedLaunch tl(0, st);
  return launch_nf4_gemm(gp, false, st);
}

hipError_t launch_linear_bwd(const LinearArgs &a, const uint16_t *X, const uint16_t *T, const uint16_t *dY,
                             const uint16_t *L1, const uint16_t *L2, uint16_t *dX, float *dL1, float *dL2,
                             void *ws, const Nf4Tables &tab, hipStream_t st) {
  const BwdLayout L = bwd_layout(a.M, a.h, a.o, a.r);
  uint16_t *sU = nullptr, *L1p = nullptr;
  GradProblem g1{}, g2{};
  float *gpart = nullptr;
  if (a.r > 0) {
    L1p = at<uint16_t>(ws, L.off_l1p);
    // U = dY·L2^T (L2 [r][o] is k-contiguous) and sU; the launch that writes them also
    // copies L1 [h][r] -> L1p [h][RP64] for the dX GEMM's rank-r step
    uint16_t *U = at<uint16_t>(ws, L.off_u);
    sU = at<uint16_t>(ws, L.off_su);
    RankParams rp{};
    rp.A = dY; rp.lda = a.o; rp.M = a.M; rp.K = a.o;
    rp.B = L2; rp.ldb = a.o; rp.r = a.r; rp.s = a.s;
    rp.out1 = U; rp.ld1 = L.RP16; rp.out2 = sU; rp.ld2 = L.RP64;
    rp.L1 = L1; rp.h = a.h; rp.ldp = L.RP64; rp.L1p = L1p;
    const hipError_t e = rank_r(rp, false, L.RP16, at<float>(ws, L.off_up), st);
    if (e != hipSuccess) return e;
    // dL1 = s·X^T·U (P = X [M][h], Q = U [M][RP16]) and dL2 = s·T^T·dY (P = dY [M][o], Q = T [M][r]), stored [r][o]
    g1 = GradProblem{X, a.h, a.h, U, L.RP16, dL1, false, cdiv(a.h, kGradTile), 0};
    g2 = GradProblem{dY, a.o, a.o, T, a.r, dL2, true, cdiv(a.o, kGradTile), a.h};
    gpart = at<float>(ws, L.off_g);
  }
  if (a.M <= 16) {
    GvdParams vp{};
    vp.dY = dY; vp.ldy = a.o; vp.M = (int)a.M;
    vp.codes = a.codes; vp.qabsmax = a.qabsmax; vp.scale2 = a.scale2; vp.mean = a.mean;
    vp.h = a.h; vp.o = a.o;
    // rows per chunk (at most L.dxc chunks; trailing ones may be empty and then store zeros)
    vp.rows = (int)rup((a.o + L.dxc - 1) / L.dxc, kGvmRows);
    vp.part = at<float>(ws, L.off_dxp);
    fill_levels(vp.level, tab);
    const dim3 grid((unsigned)((a.h + kGvdCols - 1) / kGvdCols), (unsigned)L.dxc);
    if (a.r > 0) {
      const hipError_t e = lora_grad(g1, g2, a.r, a.s, a.M, L.RP16, L.gs, gpart, st);
      if (e != hipSuccess) return e;
    }
    {
      TimedLaunch tl(1, st);
      const hipError_t e = launch(nf4_gemv_dx_kernel, grid, kGvmThreads, st, vp);
      if (e != hipSuccess) return e;
    }
    const int64_t cg = (a.h / 8 + 63) / 64;
    return launch(gemv_dx_finish_kernel, (unsigned)(a.M * cg), 256, st, (const float *)vp.part, L.dxc, (int)a.M,
                  a.h, (const uint16_t *)sU, L.RP64, L1, a.r, dX, a.h);
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
  // Everything runs in order on the caller's stream: the adapter gradients on a
  // side stream beside the dX GEMM cost the GEMM more than they saved (they share
  // the compute units and the cache hierarchy, and the stream fork and join add
  // their own gaps).
  if (a.r > 0) {
    const hipError_t e = lora_grad(g1, g2, a.r, a.s, a.M, L.RP16, L.gs, gpart, st);
    if (e != hipSuccess) return e;
  }
  TimedLaunch tl(1, st);
  return launch_nf4_gemm(gp, true, st);
}

}  // namespace ql

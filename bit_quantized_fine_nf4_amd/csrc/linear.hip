// NF4 + LoRA linear layer for gfx950: Y = X·W_hat + s·(X·L1)·L2 and its
// backward into dX, dL1, dL2 ([MC] "The algebra", Eq. 3 and Figure 1;
// [TT] §3-§4).  W_hat is never materialised in HBM: every kernel that needs
// it decodes the 4-bit codes in registers, rescales by the double-quantized
// block scale and hands bf16 values to the matrix cores.
//
// Kernels
//   rank_r_kernel        the rank-r products T = X·L1 and U = dY·L2^T in one
//                        launch each (MFMA 16x16x32, K split over the 16
//                        waves of a workgroup, fixed-order LDS sum), rounded
//                        to bf16 with the s-scaled copy the GEMM's rank-r
//                        step uses
//   nf4_gemm_kernel      fused dequant-GEMM, MFMA 32x32x16: forward
//                        (B = W_hat, K along h) and dX (B = W_hat^T, K
//                        along o); the rank-r LoRA product is added as extra
//                        K steps on the same accumulators
//   nf4_gemv_kernel      M <= 16 forward: streams the codes once, decodes a
//                        byte (two codes) per LDS lookup, applies the block
//                        scale after each 64-wide MFMA pair
//   nf4_gemv_dx_kernel   M <= 16 dX: streams the codes once in 64-row stages
//                        through LDS; 4-bit transposing reads give each lane
//                        a column's codes, a byte table yields the bf16 MFMA
//                        operand, the block scale rides on dY; one float32
//                        partial per row chunk
//   gemv_dx_finish_kernel  sums the row-chunk partials in order, adds s·U·L1^T
//   lora_grad_kernel     dL1 = s·X^T·U and dL2 = s·T^T·dY in one launch:
//                        reduction over tokens, LDS-transposed operands,
//                        split over tokens; the last split of a tile sums,
//                        scales by s and stores dL1 [h][r] or dL2 [r][o];
//                        runs before the dX GEMM on the caller's stream

#include "linear.h"
#include "gemm.h"

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

// Cross-workgroup split reduction.  Partials travel through device-coherent
// accesses (agent-scope stores and loads bypass the per-XCD L2s), so no
// device-wide cache writeback is needed: a workgroup stores its partials,
// waits until they are acknowledged, and counts itself in; the one that brings
// the count to `splits` then reads every split's partials (in split order, so
// the sum does not depend on which workgroup finishes last).
QL_DEV void store_partial(float *p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
QL_DEV float load_partial(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
QL_DEV bool last_of_splits(unsigned *cnt, unsigned splits) {
  __shared__ bool last;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // keeps the partial stores above this point
  __builtin_amdgcn_s_waitcnt(0);                           // ... and waits until they are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(cnt, 1u) == splits - 1;
  __syncthreads();
  return last;
}

// ---------------------------------------------------------------------------
// Rank-r products T = X·L1 (forward) and U = dY·L2^T (backward) in one launch
// ([MC] "The algebra", Eq. 3: the adapter's down projection; [TT] §4).  A
// workgroup owns `rows` (16, 8 or 4: enough workgroups to cover every compute
// unit; the MFMA rows past them read as zero) rows and the whole K; its 16
// waves split K into equal runs
// of 32-wide steps, accumulate with 16x16x32 MFMAs and meet in LDS, where the
// sum over the waves runs in a fixed order (deterministic, with no partial
// sums in HBM and no second launch).  A operand: lane (i, g) loads 16 bytes of
// row i at k + 8g, D steps ahead; rows past M read as zero.  B operand: the
// backward's L2 [r][o] is k-contiguous, so its fragments are 16-byte loads of
// L2 rows; the forward's L1 [h][r] is r-contiguous, so each step's 32 x r
// slab (contiguous in memory) is copied into the wave's own LDS area and
// gathered column by column.
// Outputs: out1[m][q] = bf16(sum) (zero for r <= q < ld1) and
// out2[m][q] = bf16(s * sum) (zero for q >= r).  The backward launch also
// writes the zero-padded copy L1p [h][ldp] of L1 that the dX GEMM's rank-r
// step reads, and clears the adapter-gradient split counters.
// ---------------------------------------------------------------------------
struct RankParams {
  const uint16_t *A;  // [M][lda] bf16
  int64_t lda, M, K;  // K: a multiple of 32
  const uint16_t *B;  // forward: L1 [K][r]; backward: L2 [r][ldb]
  int64_t ldb;
  int r;
  int rows;  // rows per workgroup: 16, 8 or 4
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
  unsigned *cnt;
  int ncnt;
};

constexpr int kRankWaves = 16;

template <int NT, bool KN>
__global__ __launch_bounds__(1024) void rank_r_kernel(RankParams p) {
  constexpr int D = NT <= 4 ? 4 : 2;  // steps whose loads are in flight together
  constexpr int RP = NT * 16;
  constexpr int SLAB = 32 * RP * 2;                    // bytes of one wave's L1 slab (32 rows of r <= RP)
  constexpr int RED = 16 * RP * 4;                     // bytes of one wave's partial sums
  constexpr int LDS = kRankWaves * (SLAB > RED ? SLAB : RED);
  __shared__ __attribute__((aligned(16))) char lds[LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, i16 = lane & 15;
  const int r = p.r;

  const int64_t m0 = (int64_t)blockIdx.x * p.rows;
  const int64_t mrows = p.M - m0 < p.rows ? p.M - m0 : p.rows;
  const auto rA = gv_rsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  const int voffA = (int)((i16 * p.lda + 8 * g) * 2);
  const auto rB = KN ? gv_rsrc(p.B, p.K * r * 2) : gv_rsrc(p.B, (int64_t)r * p.ldb * 2);
  const int64_t ksteps = p.K >> 5;
  const int64_t per = (ksteps + kRankWaves - 1) / kRankWaves;
  const int64_t s0 = wave * per, s1 = s0 + per < ksteps ? s0 + per : ksteps;
  char *slab = lds + wave * SLAB;

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};

  for (int64_t sb = s0; sb < s1; sb += D) {
    u32x4 a[D], b[D][NT];
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int64_t st = sb + u;
      if (st < s1) {  // wave-uniform
        const int ko = __builtin_amdgcn_readfirstlane((int)(st * 64));      // byte offset of k = 32 st
        const int so = __builtin_amdgcn_readfirstlane((int)(st * 64 * r));  // byte offset of its L1 slab
        a[u] = __builtin_amdgcn_raw_buffer_load_b128(rA, voffA, ko, 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (KN)  // 16-byte chunk lane + 64 t of the slab (64 r bytes)
            b[u][t] = __builtin_amdgcn_raw_buffer_load_b128(rB, (lane + 64 * t) * 16, so, 0);
          else     // L2 row 16 t + i16, k = 32 st + 8 g
            b[u][t] = __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(((16 * t + i16) * p.ldb + 8 * g) * 2), ko, 0);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (sb + u < s1) {
        if (KN) {
          // The slab is stored as 16-byte words and read back as bf16 values by other lanes of
          // this wave: the empty asm statements keep the compiler from moving the reads across
          // the stores (type-based alias analysis would allow it); a wave's LDS accesses execute
          // in order, so no hardware barrier is needed.
          asm volatile("" ::: "memory");
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if ((lane + 64 * t) * 16 < 64 * r) *reinterpret_cast<u32x4 *>(slab + (lane + 64 * t) * 16) = b[u][t];
          asm volatile("" ::: "memory");
          const uint16_t *sl = reinterpret_cast<const uint16_t *>(slab);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int q = 16 * t + i16;
            uint32_t w[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {  // unconditional reads inside the slab area, masked after
              const uint32_t lo = sl[(8 * g + 2 * x) * r + q], hi = sl[(8 * g + 2 * x + 1) * r + q];
              w[x] = q < r ? lo | (hi << 16) : 0u;
            }
            acc[t] = mfma16(a[u], u32x4{w[0], w[1], w[2], w[3]}, acc[t]);
          }
        } else {
#pragma unroll
          for (int t = 0; t < NT; ++t) acc[t] = mfma16(a[u], b[u][t], acc[t]);
        }
      }
    }
  }

  // the waves' sums meet in LDS: red[w][row][q], row = 4g + v, q = 16t + i16
  __syncthreads();
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[(wave * 16 + 4 * g + v) * RP + 16 * t + i16] = acc[t][v];
  __syncthreads();
  const int W = p.ld1 > p.ld2 ? p.ld1 : p.ld2;
  for (int o = tid; o < p.rows * W; o += 1024) {
    const int row = o / W, q = o % W;
    const int64_t m = m0 + row;
    if (m >= p.M) continue;
    float sum = 0.0f;
    if (q < r)
#pragma unroll
      for (int w = 0; w < kRankWaves; ++w) sum += red[(w * 16 + row) * RP + q];
    if (p.out1 && q < p.ld1) p.out1[m * p.ld1 + q] = q < r ? to_bf16(sum) : (uint16_t)0;
    if (p.out2 && q < p.ld2) p.out2[m * p.ld2 + q] = q < r ? to_bf16(p.s * sum) : (uint16_t)0;
  }
  if (p.L1p) {  // backward extras, spread over the whole grid (after the main loads: no stall in front of them)
    const int64_t gt = (int64_t)blockIdx.x * 1024 + tid, gn = (int64_t)gridDim.x * 1024;
    for (int64_t idx = gt; idx < p.h * p.ldp; idx += gn) {
      const int64_t a = idx / p.ldp, b = idx % p.ldp;
      p.L1p[idx] = b < r ? p.L1[a * r + b] : (uint16_t)0;
    }
    if (gt < p.ncnt) p.cnt[gt] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Few-token forward (M <= 16): Y[m][n] = sum_k X[m][k] W_hat[n][k] (+ LoRA).
// Pure streaming of the codes ([TT] §3 storage; [MC] "The algebra" Eq. 3 for
// the output).  A workgroup owns 64 output features and walks the whole K in
// stages of 256 weights (4 blocks): every stage (64 rows x 128 code bytes,
// 16 tokens x 512 activation bytes, 64 x 4 block scales) is fetched by all
// 256 threads with coalesced loads two stages ahead of use, parked in
// registers, then written to a double-buffered, XOR-swizzled LDS tile.
// Wave w takes block w of every stage for all 64 rows (four 16-row MFMA
// groups share one activation fragment) with 16x16x32 MFMAs, tokens being the
// MFMA rows.  The B operand is bf16(level[c]) from a byte -> bf16-pair table;
// the block scale a_hat multiplies each block's float32 partial.  The four
// waves' partial sums meet in LDS at the end.
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

constexpr int kGvRows = 64;          // output features per workgroup
constexpr int kGvKS = 256;           // weights along K per stage (4 blocks)
constexpr int kGvCodeB = kGvKS / 2;  // code bytes per row per stage
constexpr int kGvXB = kGvKS * 2;     // activation bytes per token per stage
constexpr int kGvThreads = 512;      // 8 waves: wave w takes block w%4, row groups 2(w/4), 2(w/4)+1
// Lookup table: 32 copies of the 256-entry table interleaved so that lane l
// only touches banks l%32 and l%32 + 32 (conflict-free 32-lane phases).
constexpr int kGvLutWords = 256 * 32;

struct GvStage {
  u32x4 c;     // codes: 16 bytes of the stage tile
  u32x4 x;     // activations: 16 bytes of the stage tile
  uint32_t q;  // one int8 block scale (threads < 256: row tid/4, block tid%4)
  float s2;    // its second-level scale
};

constexpr int kGvOOB = (int)0x80000000u;  // offset past every buffer: the load returns zero

// MT: token-count class (1, 4 or 16); output token 4g + v exists only for
// v < MT when MT < 4, so the block-scale FMAs for absent tokens are skipped.
template <int MT>
__global__ __launch_bounds__(kGvThreads) void nf4_gemv_kernel(GemvParams p) {
  __shared__ uint32_t lut[kGvLutWords];
  // stage tiles: codes [2][64 rows][128 B], activations [2][16 tokens][512 B];
  // reused for the cross-wave sum after the K loop
  __shared__ __attribute__((aligned(16))) uint8_t tiles[2 * kGvRows * kGvCodeB + 2 * 16 * kGvXB];
  __shared__ __attribute__((aligned(16))) float abuf[2][4 * kGvRows];
  uint8_t(*cbuf)[kGvRows * kGvCodeB] = reinterpret_cast<uint8_t(*)[kGvRows * kGvCodeB]>(tiles);
  uint8_t(*xbuf)[16 * kGvXB] = reinterpret_cast<uint8_t(*)[16 * kGvXB]>(tiles + 2 * kGvRows * kGvCodeB);
  __shared__ float lv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < 16) lv[tid] = p.level[tid];
  __syncthreads();
  for (int i = tid; i < kGvLutWords; i += kGvThreads) {
    const int e = i >> 5;  // word i = 32 e + copy
    lut[i] = pack_bf16x2(lv[e >> 4], lv[e & 15]);
  }

  const int64_t n0 = (int64_t)blockIdx.x * kGvRows;
  const int64_t rowB = p.K >> 1, nblk = p.K >> 6;
  const int nst = (int)((p.K + kGvKS - 1) / kGvKS);
  const float mu = *p.mean;
  // Buffer views: the workgroup's 64 code rows, its 64 rows of int8 scales,
  // all second-level scales, the M activation rows.  Per-thread offsets are
  // fixed; the stage advances through the scalar offset.  Codes and scales
  // past a row's end belong to the next row (or read as zero at the end of
  // the view): they are finite and always meet zero activations, because
  // activations past K (and tokens >= M) are forced to zero.
  const __amdgpu_buffer_rsrc_t rc = gv_rsrc(p.codes + n0 * rowB, kGvRows * rowB);
  const __amdgpu_buffer_rsrc_t rq = gv_rsrc(p.qabsmax + n0 * nblk, kGvRows * nblk);
  const __amdgpu_buffer_rsrc_t rs = gv_rsrc(p.scale2, ((p.N * nblk + kChunk - 1) / kChunk) * 4);
  const __amdgpu_buffer_rsrc_t rx = gv_rsrc(p.X, ((int64_t)(p.M - 1) * p.ldx + p.K) * 2);
  const int cr = tid >> 3, cp = tid & 7;  // code piece: row, 16-byte piece
  const int voc = (int)(cr * rowB) + 16 * cp;
  const int lc = (cr * 8 + (cp ^ ((cr >> 1) & 7))) * 16;
  const int xm = tid >> 5, xp = tid & 31;  // activation piece: token, 16-byte piece
  const int vox = xm < p.M ? (int)((xm * p.ldx + 8 * xp) * 2) : kGvOOB;
  const int xlim = p.K > 8 * xp ? (int)((p.K - 8 * xp + kGvKS - 1) / kGvKS) : 0;  // stages with this piece inside K
  const int lx = (xm * 32 + (xp ^ xm)) * 16;
  const bool sthr = tid < 4 * kGvRows;         // scale role (waves 0-3)
  const int srow = (tid >> 2) & 63, sblk = tid & 3;
  const int voq = (int)(srow * nblk) + sblk;
  const int64_t sbase = (n0 + srow) * nblk + sblk;
  const int la = (sblk * 16 + (srow & 15)) * 4 + (srow >> 4);  // abuf [block][n][group]

  auto load = [&](GvStage &R, int st) {
    R.c = __builtin_amdgcn_raw_buffer_load_b128(rc, voc, st * kGvCodeB, 0);
    R.x = __builtin_amdgcn_raw_buffer_load_b128(rx, st < xlim ? vox : kGvOOB, st * kGvXB, 0);
    R.q = __builtin_amdgcn_raw_buffer_load_b8(rq, sthr ? voq : kGvOOB, 4 * st, 0);
    R.s2 = __builtin_bit_cast(
        float, __builtin_amdgcn_raw_buffer_load_b32(rs, sthr ? (int)(((sbase + 4 * st) >> 8) * 4) : kGvOOB, 0, 0));
  };
  auto store = [&](const GvStage &R, int buf) {
    *reinterpret_cast<u32x4 *>(&cbuf[buf][lc]) = R.c;
    *reinterpret_cast<u32x4 *>(&xbuf[buf][lx]) = R.x;
    if (sthr) abuf[buf][la] = scale_hat((int8_t)(R.q & 0xFF), R.s2, mu);
  };
  // compute role: token / feature index within a 16x16 MFMA tile, k-group
  const int n = lane & 15, g = lane >> 4;
  const int lsel = lane & 31;
  const int blk = wave & 3, rp = wave >> 2;
  const int pcw = 2 * blk + (g >> 1);  // code piece of this block for this k-group
  const int pxa = 8 * blk + 2 * g;     // activation pieces pxa, pxa + 1
  const int la0 = (n * 32 + (pxa ^ n)) * 16, la1 = (n * 32 + ((pxa + 1) ^ n)) * 16;
  int lcode[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int row = 16 * (2 * rp + h) + n;
    lcode[h] = (row * 8 + (pcw ^ ((row >> 1) & 7))) * 16 + 8 * (g & 1);
  }
  constexpr int NV = MT < 4 ? MT : 4;
  float acc[2][NV];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[h][v] = 0.0f;
  auto compute = [&](int buf) {
    const uint8_t *cb = cbuf[buf];
    const uint8_t *xb = xbuf[buf];
    const u32x4 a0 = *reinterpret_cast<const u32x4 *>(xb + la0);
    const u32x4 a1 = *reinterpret_cast<const u32x4 *>(xb + la1);
    const f32x2 ah = *reinterpret_cast<const f32x2 *>(&abuf[buf][(blk * 16 + n) * 4 + 2 * rp]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x2 cw = *reinterpret_cast<const u32x2 *>(cb + lcode[h]);
      u32x4 bw[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const uint32_t w = e ? cw.y : cw.x;
#pragma unroll
        for (int t = 0; t < 4; ++t) bw[e][t] = lut[((w >> (8 * t)) & 0xFF) * 32 + lsel];
      }
      f32x4 part = mfma16(a0, bw[0], f32x4{0.0f, 0.0f, 0.0f, 0.0f});
      part = mfma16(a1, bw[1], part);
#pragma unroll
      for (int v = 0; v < NV; ++v) acc[h][v] = __builtin_fmaf(ah[h], part[v], acc[h][v]);
    }
  };

  // Two register stages in flight.  Every stage issues the same four loads
  // and the loop body is uniform: stages past the end read zero activations
  // (an extra stage adds exactly nothing), which keeps the number of loads in
  // flight identical on every path, so the wait before each LDS store covers
  // only the older register stage.  The scheduling fences keep the compiler
  // from interleaving the two register stages (which would make every wait
  // cover both).
  GvStage ra, rb;
  load(ra, 0);
  store(ra, 0);
  __builtin_amdgcn_sched_barrier(0);
  load(ra, 1);
  __builtin_amdgcn_sched_barrier(0);
  load(rb, 2);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    compute(0);
    store(ra, 1);
    load(ra, st + 3);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    compute(1);
    store(rb, 0);
    load(rb, st + 4);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  }

  // Cross-wave sum: acc[h][v] of wave (blk, rp) = partial Y[token 4g + v][row 16(2rp + h) + n]
  // red[block][token][row], rows padded to 68 floats: the 64 lanes of a store
  // (16 rows x 4 token groups) land in 64 distinct banks.
  constexpr int kRedLd = 68;
  static_assert(4 * 16 * kRedLd * 4 <= sizeof(tiles), "reduction fits in the stage tiles");
  float *red = reinterpret_cast<float *>(tiles);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int v = 0; v < NV; ++v) red[(blk * 16 + 4 * g + v) * kRedLd + 16 * (2 * rp + h) + n] = acc[h][v];
  __syncthreads();
  const int row = tid & 63;
  const int64_t col = n0 + row;
  for (int m = tid >> 6; m < p.M; m += kGvThreads / 64) {
    float y = red[m * kRedLd + row] + red[(16 + m) * kRedLd + row] + red[(32 + m) * kRedLd + row] +
              red[(48 + m) * kRedLd + row];
    for (int q = 0; q < p.r; ++q)
      y = __builtin_fmaf(bf16_lo(p.sT[(int64_t)m * p.ldt + q]), bf16_lo(p.L2[(int64_t)q * p.N + col]), y);
    p.Y[(int64_t)m * p.ldy + col] = to_bf16(y);
  }
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
// Q's from 2-byte gathers.  The next two slabs' loads are in flight while one
// is multiplied (two register stages, double-buffered LDS, one barrier per
// slab); loads past the token range read as zero.  The last token split of a
// tile sums the splits in split order, scales by s and stores the tile.
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
                                                        int64_t mchunk, int64_t prows, float *__restrict__ part,
                                                        unsigned *__restrict__ cnt) {
  constexpr int RP = NT * 16;
  constexpr int LP = kGradTile + 8;                   // P slab row stride (elements)
  constexpr int PCH = 64 * kGradTile / 8 / 256;       // 16-byte P chunks per thread per slab
  constexpr int QCH = (64 * RP / 8 + 255) / 256;      // 16-byte Q chunks per thread per slab (at most)
  __shared__ __attribute__((aligned(16))) uint16_t Ps[2][64 * LP];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[2][64 * RP];
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
    for (int u = 0; u < QCH; ++u)
      if (tid + 256 * u < 8 * ldq) *reinterpret_cast<u32x4 *>(&Qs[buf][(tid + 256 * u) * 8]) = S.q[u];
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
        uint32_t w[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {  // unconditional reads inside the slab (ldq <= RP), masked after
          const uint32_t lo = Qs[buf][(mk + 8 * g + 2 * x) * ldq + q];
          const uint32_t hi = Qs[buf][(mk + 8 * g + 2 * x + 1) * ldq + q];
          w[x] = q < rq ? lo | (hi << 16) : 0u;
        }
        const u32x4 bq{w[0], w[1], w[2], w[3]};
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
  float *out = part + ((int64_t)blockIdx.y * prows + pr.prow) * RP;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t i = i0 + wave * 32 + 16 * a + 4 * g + v;
        if (i < pr.I) store_partial(out + i * RP + t * 16 + c16, acc[a][t][v]);
      }
  if (!last_of_splits(cnt + blockIdx.x, gridDim.y)) return;
  const int S = (int)gridDim.y;
  for (int idx = tid; idx < kGradTile * rq; idx += 256) {
    // consecutive threads write consecutive addresses of the stored layout
    const int il = pr.trans ? idx % kGradTile : idx / rq;
    const int q = pr.trans ? idx / kGradTile : idx % rq;
    const int64_t i = i0 + il;
    if (i >= pr.I) continue;
    float sum = 0.0f;
#pragma unroll 8
    for (int k = 0; k < S; ++k) sum += load_partial(part + ((int64_t)k * prows + pr.prow + i) * RP + q);
    pr.out[pr.trans ? (int64_t)q * pr.I + i : i * rq + q] = s * sum;
  }
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

Split grad_split(int64_t M, int64_t I) {
  // about 512 workgroups: more token splits cost more in partial sums than they save
  const int64_t it = cdiv(I, kGradTile);
  int64_t S = cdiv(kTargetGroups, it);
  const int64_t msteps = cdiv(M, 64);
  S = S < 1 ? 1 : S;
  S = S > msteps ? msteps : S;
  int64_t chunk = rup(cdiv(M, S), 64);
  return {(int)cdiv(M, chunk), chunk};
}

struct FwdLayout {
  int RP16, RP64;
  size_t off_st, total;
};

FwdLayout fwd_layout(int64_t M, int64_t h, int64_t o, int r) {
  FwdLayout L{};
  if (r == 0) return L;
  L.RP16 = (int)rup(r, 16);
  L.RP64 = (int)rup(r, 64);
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += rup((int64_t)bytes, 256); return at; };
  L.off_st = take((size_t)M * L.RP64 * 2);
  L.total = off;
  return L;
}

struct BwdLayout {
  int RP16, RP64;
  Split gs;
  int dxc;  // few-token path (M <= 16): row chunks of the dX partial sums
  size_t off_u, off_su, off_l1p, off_g, off_cnt, off_dxp, total;
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
  L.gs = grad_split(M, h + o);
  L.off_u = take((size_t)M * L.RP16 * 2);
  L.off_su = take((size_t)M * L.RP64 * 2);
  L.off_l1p = take((size_t)h * L.RP64 * 2);
  L.off_g = take((size_t)L.gs.S * (h + o) * L.RP16 * 4);
  L.off_cnt = take((size_t)((h + o) / 64) * 4);
  L.total = off;
  return L;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(reinterpret_cast<char *>(ws) + off); }

void rank_r(RankParams &rp, bool kn, int RP16, hipStream_t st) {
  // the fewest rows per workgroup that still give 256 workgroups (one per compute unit)
  rp.rows = rp.M >= 16 * 256 ? 16 : (rp.M >= 8 * 256 ? 8 : 4);
  const unsigned grid = (unsigned)cdiv(rp.M, rp.rows);
  switch (RP16 / 16) {
#define QL_RK(NT)                                                                       \
  case NT:                                                                              \
    if (kn) rank_r_kernel<NT, true><<<grid, 1024, 0, st>>>(rp);                          \
    else rank_r_kernel<NT, false><<<grid, 1024, 0, st>>>(rp);                            \
    break;
    QL_RK(1) QL_RK(2) QL_RK(3) QL_RK(4) QL_RK(5) QL_RK(6) QL_RK(7) QL_RK(8)
#undef QL_RK
  }
}

void lora_grad(const GradProblem &pa, const GradProblem &pb, int r, float s, int64_t M, int RP16, const Split &sp,
               float *part, unsigned *cnt, hipStream_t st) {
  dim3 grid((unsigned)(pa.tiles + pb.tiles), (unsigned)sp.S);
  const int64_t prows = pa.I + pb.I;
  switch (RP16 / 16) {
#define QL_LG(NT)                                                                                                 \
  case NT:                                                                                                        \
    lora_grad_kernel<NT><<<grid, 256, 0, st>>>(pa, pb, r, s, M, sp.chunk, prows, part, cnt); \
    break;
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
  for (int c = w; c < chunks; c += 4) {
    const float *src = part + ((int64_t)c * M + m) * h + k;
    const f32x4 a = *reinterpret_cast<const f32x4 *>(src), b = *reinterpret_cast<const f32x4 *>(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] += a[i];
      v[4 + i] += b[i];
    }
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
    // T = X·L1 (rank r) and its s-scaled, zero-padded copy sT for the GEMM's rank-r step
    sT = at<uint16_t>(ws, L.off_st);
    RankParams rp{};
    rp.A = X; rp.lda = a.h; rp.M = a.M; rp.K = a.h;
    rp.B = L1; rp.ldb = a.r; rp.r = a.r; rp.s = a.s;
    rp.out1 = T; rp.ld1 = a.r; rp.out2 = sT; rp.ld2 = L.RP64;
    rank_r(rp, true, L.RP16, st);
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
      const unsigned grid = (unsigned)(a.o / kGvRows);
      if (a.M == 1)
        nf4_gemv_kernel<1><<<grid, kGvThreads, 0, st>>>(gp);
      else if (a.M <= 4)
        nf4_gemv_kernel<4><<<grid, kGvThreads, 0, st>>>(gp);
      else
        nf4_gemv_kernel<16><<<grid, kGvThreads, 0, st>>>(gp);
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
  GradProblem g1{}, g2{};
  float *gpart = nullptr;
  unsigned *gcnt = nullptr;
  if (a.r > 0) {
    unsigned *cnt = at<unsigned>(ws, L.off_cnt);
    L1p = at<uint16_t>(ws, L.off_l1p);
    // U = dY·L2^T (L2 [r][o] is k-contiguous) and sU; the same launch writes L1 [h][r] ->
    // L1p [h][RP64] for the dX GEMM's rank-r step and clears the gradient split counters
    uint16_t *U = at<uint16_t>(ws, L.off_u);
    sU = at<uint16_t>(ws, L.off_su);
    RankParams rp{};
    rp.A = dY; rp.lda = a.o; rp.M = a.M; rp.K = a.o;
    rp.B = L2; rp.ldb = a.o; rp.r = a.r; rp.s = a.s;
    rp.out1 = U; rp.ld1 = L.RP16; rp.out2 = sU; rp.ld2 = L.RP64;
    rp.L1 = L1; rp.h = a.h; rp.ldp = L.RP64; rp.L1p = L1p; rp.cnt = cnt; rp.ncnt = (int)((a.h + a.o) / 64);
    rank_r(rp, false, L.RP16, st);
    // dL1 = s·X^T·U (P = X [M][h], Q = U [M][RP16]) and dL2 = s·T^T·dY (P = dY [M][o], Q = T [M][r]), stored [r][o]
    g1 = GradProblem{X, a.h, a.h, U, L.RP16, dL1, false, cdiv(a.h, kGradTile), 0};
    g2 = GradProblem{dY, a.o, a.o, T, a.r, dL2, true, cdiv(a.o, kGradTile), a.h};
    gpart = at<float>(ws, L.off_g);
    gcnt = cnt;
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
    auto launch_dx = [&]() {
      {
        TimedLaunch tl(1, st);
        nf4_gemv_dx_kernel<<<grid, kGvmThreads, 0, st>>>(vp);
      }
      const int64_t cg = (a.h / 8 + 63) / 64;
      gemv_dx_finish_kernel<<<(unsigned)(a.M * cg), 256, 0, st>>>(vp.part, L.dxc, (int)a.M, a.h, sU, L.RP64, L1,
                                                                 a.r, dX, a.h);
    };
    if (a.r > 0) lora_grad(g1, g2, a.r, a.s, a.M, L.RP16, L.gs, gpart, gcnt, st);
    launch_dx();
    return hipGetLastError();
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
  if (a.r > 0) lora_grad(g1, g2, a.r, a.s, a.M, L.RP16, L.gs, gpart, gcnt, st);
  {
    TimedLaunch tl(1, st);
    launch_nf4_gemm(gp, true, st);
  }
  return hipGetLastError();
}

}  // namespace ql

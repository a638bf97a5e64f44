// Fused NF4 dequant-GEMM for gfx950 (forward and dX directions).
//
// [MC] "1. NormalFloat" / [GO] "The core move": the 4-bit weights are
// dequantized to BF16 on the fly for the matrix multiplication and never
// stored in wider form.  Here every workgroup decodes the codes of its weight
// tile straight into LDS as bf16(level[code] * a_hat) and feeds bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with float32 accumulation.
//
// Layout.  256 threads = 2 x 2 waves, workgroup tile BM x BN, K step 64.
//  A tile  [m][k] in LDS (row stride 72 bf16), read as 16-byte fragments.
//  Forward B tile [n][k] (row stride 72): each 32-weight unit is one half of
//   one 64-weight block of codes row n, i.e. one scale per unit.
//  dX B tile [k][n] (row stride BN + 16): the codes are contiguous along n
//   (h), so each unit is 32 consecutive n of one row k — again one scale per
//   unit — and the MFMA B fragments (8 consecutive k of one n) come from two
//   transposing LDS reads (ds_read_b64_tr_b16).  A 16-lane group of that
//   instruction returns, to lane i, element i%4 of the 8-byte chunks named by
//   lanes i/4, 4+i/4, 8+i/4, 12+i/4; lane 4j+q names row k0+j, column n0+4q,
//   so lane i receives rows k0..k0+3 of column n0+i.
// Decoding.  A 256-entry table at LDS offset 0 maps a code byte to the pair
//  (level[high nibble], level[low nibble]); one shifted byte gives the table
//  address, one 8-byte LDS read gives both levels, two multiplies by a_hat and
//  one packed convert give the two bf16 weights.
// Loads.  All global reads are raw buffer loads with per-tile descriptors:
//  rows past the end of a matrix read as zero, so there are no branches and
//  no 64-bit address arithmetic in the K loop.
// LoRA.  The rank-r term s·(X·L1)·L2 (forward) or s·(dY·L2^T)·L1^T (dX) is
//  added by extra K steps over (A2, B2) on the same accumulators.

#include "gemm.h"

namespace ql {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

QL_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
QL_DEV u32x4 bload128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
QL_DEV int8_t bload_i8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return (int8_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}
QL_DEV float bload_f32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
QL_DEV f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                0, 0);
}
QL_DEV u32x4 tr_pair(const uint16_t *lo, const uint16_t *hi) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lo));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(hi));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}
QL_DEV uint16_t to_bf16(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

}  // namespace

template <int BM, int BN, bool TRANS>
__global__ __launch_bounds__(256) void nf4_gemm_kernel(GemmParams p) {
  constexpr int BK = 64;
  constexpr int LDA = BK + 8;    // A [m][k]
  constexpr int LDNK = BK + 8;   // B [n][k]
  constexpr int LDKN = BN + 16;  // B [k][n]
  constexpr int B_ELEMS = (BN * LDNK > BK * LDKN) ? BN * LDNK : BK * LDKN;
  constexpr int STAGE = BM * LDA + B_ELEMS;
  constexpr int WTM = BM / 2, WTN = BN / 2, TM = WTM / 32, TN = WTN / 32;
  constexpr int A_CH = BM * 8 / 256;   // 16-byte A chunks per thread per K step
  constexpr int WU = BN / 128;         // 32-weight units per thread per K step
  constexpr int B2_CH = BN * 8 / 256;  // 16-byte LoRA-B chunks per thread
  constexpr int LUT_BYTES = 256 * 8;
  static_assert(2 * STAGE >= BM * (BN + 8), "epilogue staging must fit");
  __shared__ __attribute__((aligned(16))) char lds[LUT_BYTES + 2 * STAGE * 2];
  const f32x2 *lut = reinterpret_cast<const f32x2 *>(lds);
  uint16_t *smem = reinterpret_cast<uint16_t *>(lds + LUT_BYTES);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  reinterpret_cast<f32x2 *>(lds)[tid] = f32x2{p.level[tid >> 4], p.level[tid & 15]};

  int bid = blockIdx.x;
  const int ntiles = p.tiles_m * p.tiles_n;
  if ((ntiles & 7) == 0) bid = (bid & 7) * (ntiles >> 3) + (bid >> 3);  // one XCD -> contiguous tiles
  const int tn = bid % p.tiles_n, tm = bid / p.tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t mrows = p.M - m0 < BM ? p.M - m0 : BM;
  const int64_t nrows = p.N - n0 < BN ? p.N - n0 : BN;
  const float mu = *p.mean;
  const int64_t bpr = p.ldw >> 6;  // 64-blocks per codes row

  const auto rA = make_rsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  const auto rS2 = make_rsrc(p.scale2, ((p.wrows * bpr + 255) >> 8) * 4);

  // per-thread constant offsets
  int voffA[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int chunk = tid + 256 * c;
    voffA[c] = (int)(((chunk >> 3) * p.lda + (chunk & 7) * 8) * 2);
  }
  int voffC[WU], voffQ[WU];
  int64_t blk0[WU];
#pragma unroll
  for (int u = 0; u < WU; ++u) {
    const int unit = tid + 256 * u;
    if (!TRANS) {
      const int row = unit >> 1, half = unit & 1;
      voffC[u] = (int)(row * (p.ldw >> 1) + half * 16);
      voffQ[u] = (int)(row * bpr);
      blk0[u] = (n0 + row) * bpr;
    } else {
      const int krow = unit / (BN / 32), part = unit % (BN / 32);
      voffC[u] = (int)(krow * (p.ldw >> 1) + part * 16);
      voffQ[u] = (int)(krow * bpr + (part >> 1));
      blk0[u] = krow * bpr + ((n0 + part * 32) >> 6);
    }
  }
  const auto rCf = make_rsrc(p.codes + n0 * (p.ldw >> 1), nrows * (p.ldw >> 1));
  const auto rQf = make_rsrc(p.qabsmax + n0 * bpr, nrows * bpr);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  auto As = [&](int buf) { return smem + buf * STAGE; };
  auto Bs = [&](int buf) { return smem + buf * STAGE + BM * LDA; };

  u32x4 ra[A_CH];
  u32x4 rc[WU];
  int8_t rq[WU];
  float rs[WU];

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) ra[c] = bload128(rA, voffA[c], kt * BK * 2);
    if (!TRANS) {
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        rc[u] = bload128(rCf, voffC[u], kt * 32);
        rq[u] = bload_i8(rQf, voffQ[u], kt);
        rs[u] = bload_f32(rS2, (int)(((blk0[u] + kt) >> 8) * 4), 0);
      }
    } else {
      const int64_t krow0 = (int64_t)kt * BK;
      const auto rC = make_rsrc(p.codes + krow0 * (p.ldw >> 1) + (n0 >> 1),
                                (p.wrows - krow0) * (p.ldw >> 1) - (n0 >> 1));
      const auto rQ = make_rsrc(p.qabsmax + krow0 * bpr + (n0 >> 6), (p.wrows - krow0) * bpr - (n0 >> 6));
#pragma unroll
      for (int u = 0; u < WU; ++u) {
        rc[u] = bload128(rC, voffC[u], 0);
        rq[u] = bload_i8(rQ, voffQ[u], 0);
        rs[u] = bload_f32(rS2, (int)(((blk0[u] + krow0 * bpr) >> 8) * 4), 0);
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t *as = As(buf);
    uint16_t *bs = Bs(buf);
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int chunk = tid + 256 * c;
      *reinterpret_cast<u32x4 *>(as + (chunk >> 3) * LDA + (chunk & 7) * 8) = ra[c];
    }
#pragma unroll
    for (int u = 0; u < WU; ++u) {
      const int unit = tid + 256 * u;
      const float ah = scale_hat(rq[u], rs[u], mu);
      uint32_t o[16];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x2 l = lut[(rc[u][d] >> (8 * b)) & 0xFF];
          o[4 * d + b] = pack_bf16x2(l[0] * ah, l[1] * ah);
        }
      uint16_t *dst;
      if (!TRANS) {
        dst = bs + (unit >> 1) * LDNK + (unit & 1) * 32;
      } else {
        dst = bs + (unit / (BN / 32)) * LDKN + (unit % (BN / 32)) * 32;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        reinterpret_cast<u32x4 *>(dst)[q] = u32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    }
  };

  // kn = true: B tile is [k][n] (transposing reads); false: [n][k] (plain 16-byte reads)
  auto compute = [&](int buf, bool kn) {
    const uint16_t *as = As(buf) + (wm * WTM + (lane & 31)) * LDA + (lane >> 5) * 8;
    const uint16_t *bsb = Bs(buf);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      u32x4 af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) af[i] = *reinterpret_cast<const u32x4 *>(as + i * 32 * LDA + kk * 16);
      if (!kn) {
        const uint16_t *bs = bsb + (wn * WTN + (lane & 31)) * LDNK + (lane >> 5) * 8 + kk * 16;
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const u32x4 *>(bs + j * 32 * LDNK);
      } else {
        const int c = lane & 15;
        const int kb = kk * 16 + (lane >> 5) * 8 + (c >> 2);
        const uint16_t *bs = bsb + kb * LDKN + wn * WTN + ((lane >> 4) & 1) * 16 + (c & 3) * 4;
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = tr_pair(bs + j * 32, bs + 4 * LDKN + j * 32);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  };

  __syncthreads();  // decode table ready
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < p.ksteps; ++kt) {
    const bool more = kt + 1 < p.ksteps;
    if (more) load_tile(kt + 1);
    compute(kt & 1, TRANS);
    if (more) store_tile((kt + 1) & 1);
    __syncthreads();
  }

  // LoRA K steps.  Forward: B2 = L2 [r][N] read as a [k][n] tile; dX: B2 = L1 padded
  // to [N][ldb2] read as an [n][k] tile.  Rows past the ends read as zero.
  if (p.ksteps2 > 0) {
    const auto rA2 = make_rsrc(p.A2 + m0 * p.lda2, mrows * p.lda2 * 2);
    const auto rB2 = TRANS ? make_rsrc(p.B2 + n0 * p.ldb2, nrows * p.ldb2 * 2)
                           : make_rsrc(p.B2 + n0, ((int64_t)p.b2rows * p.ldb2 - n0) * 2);
    for (int k2 = 0; k2 < p.ksteps2; ++k2) {
      uint16_t *as = As(0);
      uint16_t *bs = Bs(0);
#pragma unroll
      for (int c = 0; c < A_CH; ++c) {
        const int chunk = tid + 256 * c, row = chunk >> 3, col8 = chunk & 7;
        *reinterpret_cast<u32x4 *>(as + row * LDA + col8 * 8) =
            bload128(rA2, (int)((row * p.lda2 + col8 * 8) * 2), k2 * BK * 2);
      }
#pragma unroll
      for (int c = 0; c < B2_CH; ++c) {
        const int chunk = tid + 256 * c;
        if (TRANS) {  // [n][k] tile: BN rows of 8 chunks
          const int row = chunk >> 3, col8 = chunk & 7;
          *reinterpret_cast<u32x4 *>(bs + row * LDNK + col8 * 8) =
              bload128(rB2, (int)((row * p.ldb2 + col8 * 8) * 2), k2 * BK * 2);
        } else {  // [k][n] tile: 64 rows of BN/8 chunks
          const int krow = chunk / (BN / 8), col8 = chunk % (BN / 8);
          *reinterpret_cast<u32x4 *>(bs + krow * LDKN + col8 * 8) =
              bload128(rB2, (int)(((int64_t)(k2 * BK + krow) * p.ldb2 + col8 * 8) * 2), 0);
        }
      }
      __syncthreads();
      compute(0, !TRANS);
      __syncthreads();
    }
  }

  // Epilogue: fp32 -> bf16 through LDS, then coalesced 16-byte stores.
  constexpr int LDC = BN + 8;
  uint16_t *cs = smem;
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WTM + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = wn * WTN + 32 * j + (lane & 31);
        cs[row * LDC + col] = to_bf16(acc[i][j][v]);
      }
  __syncthreads();
  for (int chunk = tid; chunk < BM * BN / 8; chunk += 256) {
    const int row = chunk / (BN / 8), c8 = chunk % (BN / 8);
    const int64_t m = m0 + row, n = n0 + c8 * 8;
    if (m < p.M && n < p.N)
      *reinterpret_cast<u32x4 *>(p.C + m * p.ldc + n) = *reinterpret_cast<const u32x4 *>(cs + row * LDC + c8 * 8);
  }
}

namespace {

inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

template <int BM, int BN, bool TRANS>
void gemm_launch(GemmParams &gp, hipStream_t st) {
  gp.tiles_m = (int)cdiv(gp.M, BM);
  gp.tiles_n = (int)cdiv(gp.N, BN);
  nf4_gemm_kernel<BM, BN, TRANS><<<gp.tiles_m * gp.tiles_n, 256, 0, st>>>(gp);
}

template <bool TRANS>
void gemm_select(GemmParams &gp, hipStream_t st) {
  const int64_t t256 = cdiv(gp.M, 256) * cdiv(gp.N, 256);
  const int64_t t256x128 = cdiv(gp.M, 256) * cdiv(gp.N, 128);
  if (gp.M >= 256 && t256 >= 240) gemm_launch<256, 256, TRANS>(gp, st);
  else if (gp.M >= 256 && t256x128 >= 200) gemm_launch<256, 128, TRANS>(gp, st);
  else gemm_launch<128, 128, TRANS>(gp, st);
}

}  // namespace

void launch_nf4_gemm(GemmParams &gp, bool trans, hipStream_t st) {
  if (trans) gemm_select<true>(gp, st);
  else gemm_select<false>(gp, st);
}

}  // namespace ql

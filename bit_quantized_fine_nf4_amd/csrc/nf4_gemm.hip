// Fused NF4 dequant-GEMM for gfx950 (forward and dX directions).
//
// [MC] "1. NormalFloat" / [GO] "The core move": the 4-bit weights are
// dequantized to BF16 on the fly for the matrix multiplication and never
// stored in wider form.  Every workgroup decodes the codes of its weight tile
// straight into LDS as bf16(level[code] * a_hat) and feeds bf16 MFMA
// (v_mfma_f32_32x32x16_bf16) with float32 accumulation.
//
// Workgroup: 512 threads = 4 x 2 waves (two waves per SIMD, so one wave's
// matrix-core work overlaps the other's LDS and decode work), tile BM x BN,
// K step 64, wave tile (BM/4) x (BN/2).  Both operands are staged through
// double-buffered LDS; later K steps' global loads are in flight while the
// matrix cores work on the current buffers.  Within a K step, lane group
// g = lane/32 owns k in [32g, 32g+32) and MFMA kk takes k = 32g + 8kk + 0..7
// (the contraction may visit k in any order as long as A and B agree).
// The tiles are 256 x 128 and 128 x 128 (256 x 256 tiles, in both directions,
// run the four-wave kernels of nf4_gemm_wide.hip).
//  A operand (X or dY, k-contiguous): tile [m][k].  It goes from memory straight
//   into LDS (buffer_load ... lds, 16 bytes per lane, 1 KB = 8 rows per
//   instruction) one step ahead, in unpadded 128-byte rows whose 16-byte chunks
//   are XOR-swizzled by row so fragment reads stay free of bank conflicts.
//  B operand is decoded into LDS:
//   Every thread decodes one unit of 16 consecutive weights of one codes row
//   per K step (inside one 64-weight block, so one scale per unit).
//   forward: tile [n][k] (row stride 72), units along k of codes row n;
//    fragments are 16-byte LDS reads.
//   dX: tile [k][n] (row stride BN + 16); codes are contiguous along n (h),
//    units run along n of one row k; fragments
//    (8 consecutive k of one n) come from two transposing LDS reads
//    (ds_read_b64_tr_b16).  In each 16-lane group that instruction returns to
//    lane i element i%4 of the 8-byte chunks named by lanes i/4, 4+i/4, 8+i/4,
//    12+i/4; lane 4j+q names row k0+j, column n0+4q, so lane i receives rows
//    k0..k0+3 of column n0+i.
// Decoding: a 256-entry table at LDS offset 0 maps a code byte to the pair
//  (level[high nibble], level[low nibble]); one shifted byte gives the table
//  address, one 8-byte LDS read gives both levels, two multiplies by a_hat and
//  one packed convert give the two bf16 weights.  The 256x128 tiles keep 16
//  interleaved copies of the table (lane l reads copy l % 16) against bank
//  conflicts.
// Loads: raw buffer loads with per-tile descriptors — rows past the end of a
//  matrix read as zero, so the K loop has no branches and no 64-bit address
//  arithmetic.
// LoRA: the rank-r term s·(X·L1)·L2 (forward) or s·(dY·L2^T)·L1^T (dX) is added
//  by extra K steps over (A2, B2) on the same accumulators.

#include "gemm.h"

#include <type_traits>

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
// 16 bytes per lane from a buffer straight into LDS (buffer_load ... lds): lane L's
// bytes land at dst + 16 L; dst must be the same in every lane of the wave.
QL_DEV void load16_to_lds(__amdgpu_buffer_rsrc_t r, uint16_t *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

}  // namespace

template <int BM, int BN, bool TRANS>
__global__ __launch_bounds__(512) void nf4_gemm_kernel(GemmParams p) {
  constexpr int NT = 512, BK = 64;
  constexpr int WTM = BM / 4, WTN = BN / 2, TM = WTM / 32, TN = WTN / 32;
  static_assert(BN == 128 && (BM == 256 || BM == 128), "256 x 128 or 128 x 128 tiles");
  constexpr int LDA = BK;        // A [m][k]: unpadded rows of swizzled chunks
  constexpr int LDNK = BK + 8;   // B [n][k]
  // B [k][n] row stride: 16 banks (mod 64), so the 32 lanes of a transposing
  // fragment read (4 rows x 2 groups of 4 eight-byte chunks) cover the 64 banks
  // once.  The decode stores (2 rows of 16-byte units per 16 lanes) then pair
  // up, but they are 8x rarer.  Against a 12-bank stride: dX GEMM on a
  // 4096 x 4096 weight with 2048 tokens 93.8 -> 90.6 us.
  constexpr int LDKN = BN + 32;
  constexpr int B_ELEMS = cmax(BN * LDNK, BK * LDKN);
  constexpr int STAGE = BM * LDA + B_ELEMS;  // elements per LDS stage (A then B)
  constexpr int UW = 64 * BN / NT;  // weights per decode unit (16): every thread decodes one unit
  constexpr int UB = UW / 2;        // code bytes per unit (8)
  constexpr int A_CH = BM * 8 / NT;  // 16-byte A chunks per thread per K step
  // Interleaved copies of the decode table: lane l reads copy l % LUT_COPIES,
  // which cuts the bank conflicts of the random code-byte reads.  The 256x128
  // tiles have the LDS for 16 copies (dX GEMM on a 4096 x 4096 weight with 2048
  // tokens 97.7 -> 93.8 us; a conflict-free timing knob reaches 92.8).
  constexpr int LUT_COPIES = BM == 256 ? 16 : 1;
  constexpr int LUT_BYTES = 256 * 8 * LUT_COPIES;
  constexpr int LDC = BN + 8;
  constexpr int LDS_BYTES = cmax(LUT_BYTES + 2 * STAGE * 2, BM * LDC * 2);
  static_assert(A_CH >= 1, "A tile too small");
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  const f32x2 *lut = reinterpret_cast<const f32x2 *>(lds);
  uint16_t *sm = reinterpret_cast<uint16_t *>(lds + LUT_BYTES);
  uint16_t *bsm = sm + BM * LDA;  // B tile of stage 0 (stage 1 is STAGE elements further)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // row r keeps its 8 chunks of 16 bytes in the order c ^ aswz(r), so the 16 lanes of a
  // fragment read (16 rows, one chunk) hit 16 different 16-byte bank groups without padding.
  auto a_off = [](int r, int chunk) { return r * LDA + ((chunk ^ ((r >> 1) & 7)) << 3); };
  for (int i = tid; i < 256 * LUT_COPIES; i += NT) {
    const int e = i / LUT_COPIES;
    reinterpret_cast<f32x2 *>(lds)[i] = f32x2{p.level[e >> 4], p.level[e & 15]};
  }

  int tm, tn;
  gemm_tile_of(blockIdx.x, p.tiles_m, p.tiles_n, 2, tm, tn);
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t mrows = p.M - m0 < BM ? p.M - m0 : BM;
  const int64_t nrows = p.N - n0 < BN ? p.N - n0 : BN;
  const float mu = *p.mean;
  const int64_t bpr = p.ldw >> 6;  // 64-blocks per codes row
  const int g = lane >> 5, l32 = lane & 31;

  // ---- A tile ----
  // Each wave loads A_CH blocks of 8 rows into LDS, one 1 KB block per instruction, so
  // lane L fetches the global chunk that belongs at row 8 rb + L / 8, physical chunk L % 8.
  const auto rA = make_rsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  int voffA[A_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int r = 8 * (wv * A_CH + c) + (lane >> 3), lc = (lane & 7) ^ ((r >> 1) & 7);
    voffA[c] = (int)((r * p.lda + lc * 8) * 2);
  }
  auto load_a_lds = [&](int kt_, int buf) {
    const int kt = __builtin_amdgcn_readfirstlane(kt_);
#pragma unroll
    for (int c = 0; c < A_CH; ++c) load16_to_lds(rA, sm + buf * STAGE + (wv * A_CH + c) * 8 * LDA, voffA[c], kt * BK * 2);
  };

  // ---- B decode unit of this thread: UW consecutive weights of one codes row ----
  int voffC = 0, voffQ = 0;
  int64_t blk0 = 0;
  uint16_t *bdst0;  // LDS destination of the unit (buffer 0)
  if (!TRANS) {
    constexpr int PER_ROW = 64 / UW;  // units per 64-weight block
    const int row = tid / PER_ROW, part = tid % PER_ROW;
    voffC = (int)(row * (p.ldw >> 1) + part * UB);
    voffQ = (int)(row * bpr);
    blk0 = (n0 + row) * bpr;
    bdst0 = bsm + row * LDNK + part * UW;
  } else {
    constexpr int PER_ROW = BN / UW;  // units per tile row
    const int krow = tid / PER_ROW, part = tid % PER_ROW;
    voffC = (int)(krow * (p.ldw >> 1) + part * UB);
    voffQ = (int)(krow * bpr + ((part * UW) >> 6));
    blk0 = krow * bpr + ((n0 + part * UW) >> 6);
    bdst0 = bsm + krow * LDKN + part * UW;
  }
  const auto rS2 = make_rsrc(p.scale2, ((p.wrows * bpr + 255) >> 8) * 4);
  const auto rCf = make_rsrc(p.codes + n0 * (p.ldw >> 1), nrows * (p.ldw >> 1));
  const auto rQf = make_rsrc(p.qabsmax + n0 * bpr, nrows * bpr);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // One register set holds everything a K step needs from global memory.
  struct Stage {
    u32x4 c;        // this thread's code bytes (UB of them)
    uint32_t q;     // its int8 block scale, zero-extended (see put_part)
    float s2;       // its second-level scale
  };
  auto load_stage = [&](int kt_, Stage &S) {
    // The step index is wave-uniform; saying so keeps the scalar offsets in SGPRs
    // (otherwise every buffer load becomes a per-lane waterfall loop).
    const int kt = __builtin_amdgcn_readfirstlane(kt_);
    if (!TRANS) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rCf, voffC, kt * 32, 0);
      S.c = u32x4{v[0], v[1], 0u, 0u};
      S.q = __builtin_amdgcn_raw_buffer_load_b8(rQf, voffQ, kt, 0);
      S.s2 = bload_f32(rS2, (int)(((blk0 + kt) >> 8) * 4), 0);
    } else {
      const int64_t krow0 = (int64_t)kt * BK;
      const auto rC = make_rsrc(p.codes + krow0 * (p.ldw >> 1) + (n0 >> 1),
                                (p.wrows - krow0) * (p.ldw >> 1) - (n0 >> 1));
      const auto rQ = make_rsrc(p.qabsmax + krow0 * bpr + (n0 >> 6), (p.wrows - krow0) * bpr - (n0 >> 6));
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rC, voffC, 0, 0);
      S.c = u32x4{v[0], v[1], 0u, 0u};
      S.q = __builtin_amdgcn_raw_buffer_load_b8(rQ, voffQ, 0, 0);
      S.s2 = bload_f32(rS2, (int)(((blk0 + krow0 * bpr) >> 8) * 4), 0);
    }
  };
  // Part `part` (0..3) of writing a stage's B into LDS buffer `buf`: a quarter of
  // the code bytes, decoded (LUT pair -> * a_hat -> bf16) and stored.  `ah` is the
  // stage's block scale (computed by part 0).
  constexpr int BPP = UB / 4;  // code bytes decoded per part (2)
  // All eight table reads of a step are issued at its start (right after the next
  // stage's loads), so their LDS latency is paid once rather than once per part.
  const int lcopy = lane % LUT_COPIES;
  auto lut_index = [&](uint32_t w) { return (int)(w & 0xFF) * LUT_COPIES + lcopy; };
  f32x2 LV[UB];
  auto read_levels = [&](const Stage &S) {
#pragma unroll
    for (int byte = 0; byte < UB; ++byte) LV[byte] = lut[lut_index(S.c[byte >> 2] >> (8 * (byte & 3)))];
  };
  uint32_t oprev[2] = {0u, 0u};  // an even part's decoded words, stored with the next part's
  auto put_part = [&](int buf, int part, const Stage &S, float &ah) {
    // int8 value from the zero-extended byte by float arithmetic: a plain
    // sign extension would let instruction selection fuse it with the load
    // and move that load to this point, next to the younger prefetch.
    if (part == 0) {
      const float qf = (float)S.q - (float)(S.q & 0x80u) * 2.0f;
      ah = qf * S.s2 + mu;
    }
    uint32_t o[BPP];
#pragma unroll
    for (int b = 0; b < BPP; ++b) {
      const f32x2 l = LV[part * BPP + b];
      o[b] = pack_bf16x2(l[0] * ah, l[1] * ah);
    }
    // two parts per 16-byte store: even parts keep their words, odd parts store both
    uint16_t *dst = bdst0 + buf * STAGE + part * 2 * BPP;
    if (part & 1)
      *reinterpret_cast<u32x4 *>(dst - 2 * BPP) = u32x4{oprev[0], oprev[1], o[0], o[1]};
    else
      oprev[0] = o[0], oprev[1] = o[1];
  };
  // B fragments of MFMA step kk from an LDS tile; kn: tile is [k][n] (transposing reads)
  auto load_bfrag = [&](const uint16_t *bs, bool kn, int kk, u32x4 (&bf)[TN]) {
    if (!kn) {
      const uint16_t *b0 = bs + (wn * WTN + l32) * LDNK + 32 * g + 8 * kk;
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const u32x4 *>(b0 + j * 32 * LDNK);
    } else {
      const int c = lane & 15;
      const uint16_t *b0 = bs + (32 * g + 8 * kk + (c >> 2)) * LDKN + wn * WTN + ((lane >> 4) & 1) * 16 + (c & 3) * 4;
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[j] = tr_pair(b0 + j * 32, b0 + 4 * LDKN + j * 32);
    }
  };
  // Fragments of MFMA group kk (A: TM, B: TN 16-byte pieces per lane).
  struct Frags {
    u32x4 a[TM], b[TN];
  };
  auto load_frags = [&](int buf, bool kn, int kk, Frags &F) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      F.a[i] = *reinterpret_cast<const u32x4 *>(sm + buf * STAGE + a_off(wm * WTM + i * 32 + l32, 4 * g + kk));
    load_bfrag(bsm + buf * STAGE, kn, kk, F.b);
  };
  auto mma_frags = [&](const Frags &F) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(F.a[i], F.b[j], acc[i][j]);
  };
  auto mma_kk = [&](int buf, bool kn, int kk) {
    Frags F;
    load_frags(buf, kn, kk, F);
    mma_frags(F);
  };
  auto mma_step = [&](int buf, bool kn) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma_kk(buf, kn, kk);
  };

  // Software pipeline.  Step kt computes on LDS buffer kt&1 while, between its
  // four MFMA groups, the next step's A chunks and decoded B are written into
  // the other buffer from registers loaded one step earlier, and the loads for
  // step kt+2 are in flight.  One barrier per step.  Loads past the last step
  // read harmless data (zeros or the next row) that is never used.
  Stage S0, S1;
  float ah = 0.0f;
  __syncthreads();  // decode table ready
  const int nk = p.ksteps;
  // LoRA K steps.  Forward: B2 = L2 [r][N] read as a [k][n] tile; dX: B2 = L1 padded
  // to [N][ldb2] read as an [n][k] tile.  Rows past the ends read as zero (and every
  // load reads zero when there is no LoRA term: the resources are then empty).
  constexpr int B2CH = BN * 8 / NT;  // 16-byte B2 chunks per thread per LoRA step
  const bool lora = p.ksteps2 > 0;
  const auto rA2 = make_rsrc(p.A2 + m0 * p.lda2, lora ? mrows * p.lda2 * 2 : 0);
  const auto rB2 = TRANS ? make_rsrc(p.B2 + n0 * p.ldb2, lora ? nrows * p.ldb2 * 2 : 0)
                         : make_rsrc(p.B2 + n0, lora ? ((int64_t)p.b2rows * p.ldb2 - n0) * 2 : 0);
  struct LoraStage {
    u32x4 a[A_CH], b[B2CH];
  };
  auto lora_load = [&](int k2, LoraStage &L) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int chunk = tid + NT * c, row = chunk >> 3, col8 = chunk & 7;
      L.a[c] = bload128(rA2, (int)((row * p.lda2 + col8 * 8) * 2), k2 * BK * 2);
    }
#pragma unroll
    for (int c = 0; c < B2CH; ++c) {
      const int chunk = tid + NT * c;
      if (TRANS) {  // [n][k] tile: BN rows of 8 chunks
        const int row = chunk >> 3, col8 = chunk & 7;
        L.b[c] = bload128(rB2, (int)((row * p.ldb2 + col8 * 8) * 2), k2 * BK * 2);
      } else {  // [k][n] tile: 64 rows of BN/8 chunks
        const int krow = chunk / (BN / 8), col8 = chunk % (BN / 8);
        L.b[c] = bload128(rB2, (int)(((int64_t)(k2 * BK + krow) * p.ldb2 + col8 * 8) * 2), 0);
      }
    }
  };
  auto lora_put = [&](const LoraStage &L) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int chunk = tid + NT * c, row = chunk >> 3, col8 = chunk & 7;
      *reinterpret_cast<u32x4 *>(sm + a_off(row, col8)) = L.a[c];
    }
#pragma unroll
    for (int c = 0; c < B2CH; ++c) {
      const int chunk = tid + NT * c;
      if (TRANS) {
        const int row = chunk >> 3, col8 = chunk & 7;
        *reinterpret_cast<u32x4 *>(bsm + row * LDNK + col8 * 8) = L.b[c];
      } else {
        const int krow = chunk / (BN / 8), col8 = chunk % (BN / 8);
        *reinterpret_cast<u32x4 *>(bsm + krow * LDKN + col8 * 8) = L.b[c];
      }
    }
  };
  // the first LoRA step's operands: the oldest loads, done long before they are used
  LoraStage L0;
  lora_load(0, L0);

  // wait until at most n vector-memory operations of this wave are outstanding
  // (the LDS-bound A loads count; the compiler cannot know that other waves read them)
  auto wait_vm = [](auto nconst) {
    constexpr int n = decltype(nconst)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  };
  load_a_lds(0, 0);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(0, S0);
  __builtin_amdgcn_sched_barrier(0);
  load_stage(1, S1);
  __builtin_amdgcn_sched_barrier(0);
  read_levels(S0);
#pragma unroll
  for (int part = 0; part < 4; ++part) put_part(0, part, S0, ah);
  wait_vm(std::integral_constant<int, 3>{});  // stage 0's A, and everything older than stage 1's codes
  __syncthreads();
  auto step = [&](int kt, Stage &Snext, Stage &Sfree) {
    // Snext holds step kt+1; Sfree is refilled with step kt+2 (past the last step
    // these loads and writes are harmless and unused).  The fragments of MFMA
    // group kk+1 are read while group kk's MFMAs run.
    const int buf = kt & 1;
    load_a_lds(kt + 1, buf ^ 1);  // that buffer is read by nobody since the last barrier
    __builtin_amdgcn_sched_barrier(0);
    load_stage(kt + 2, Sfree);
    __builtin_amdgcn_sched_barrier(0);
    read_levels(Snext);
    __builtin_amdgcn_sched_barrier(0);
    Frags F0, F1;
    load_frags(buf, TRANS, 0, F0);
    load_frags(buf, TRANS, 1, F1);
    mma_frags(F0);
    put_part(buf ^ 1, 0, Snext, ah);
    load_frags(buf, TRANS, 2, F0);
    mma_frags(F1);
    put_part(buf ^ 1, 1, Snext, ah);
    load_frags(buf, TRANS, 3, F1);
    mma_frags(F0);
    put_part(buf ^ 1, 2, Snext, ah);
    mma_frags(F1);
    put_part(buf ^ 1, 3, Snext, ah);
    wait_vm(std::integral_constant<int, 3>{});  // stage kt+1's A in LDS; stage kt+2's codes may fly
    __syncthreads();
  };
  // Uniform two-step body (the same loads in flight on every path); an odd
  // last step is peeled.
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, S1, S0);
    step(kt + 1, S0, S1);
  }
  if (kt < nk) mma_step(kt & 1, TRANS);
  __builtin_amdgcn_s_waitcnt(0);  // no LDS-bound load of a stage past the end may still land
  __syncthreads();

  // LoRA K steps (after the main loop, on the same accumulators).  The first one's
  // operands were loaded in the prologue (lora_load above) where registers allow.
  for (int k2 = 0; k2 < p.ksteps2; ++k2) {
    LoraStage L;
    if (k2 == 0) L = L0;
    else lora_load(k2, L);
    lora_put(L);
    __syncthreads();
    mma_step(0, !TRANS);
    __syncthreads();
  }

  // Epilogue: fp32 -> bf16 through LDS, then coalesced 16-byte stores.
  uint16_t *cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wm * WTM + 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        const int col = wn * WTN + 32 * j + l32;
        cs[row * LDC + col] = to_bf16(acc[i][j][v]);
      }
  __syncthreads();
  for (int chunk = tid; chunk < BM * BN / 8; chunk += NT) {
    const int row = chunk / (BN / 8), c8 = chunk % (BN / 8);
    const int64_t m = m0 + row, n = n0 + c8 * 8;
    if (m < p.M && n < p.N)
      *reinterpret_cast<u32x4 *>(p.C + m * p.ldc + n) = *reinterpret_cast<const u32x4 *>(cs + row * LDC + c8 * 8);
  }
}

namespace {

inline int64_t cdiv(int64_t x, int64_t m) { return (x + m - 1) / m; }

template <int BM, int BN, bool TRANS>
hipError_t gemm_launch(GemmParams &gp, hipStream_t st) {
  gp.tiles_m = (int)cdiv(gp.M, BM);
  gp.tiles_n = (int)cdiv(gp.N, BN);
  return launch(nf4_gemm_kernel<BM, BN, TRANS>, gp.tiles_m * gp.tiles_n, 512, st, gp);
}

template <bool TRANS>
hipError_t gemm_select(GemmParams &gp, hipStream_t st) {
  const int64_t t256 = cdiv(gp.M, 256) * cdiv(gp.N, 256);
  const int64_t t256x128 = cdiv(gp.M, 256) * cdiv(gp.N, 128);
  if (gp.M >= 256 && t256 >= 240) return launch_nf4_gemm_wide(gp, TRANS, 256, st);
  // 256x128: the four-wave forward (75 against 79 us on a 4096 x 4096 weight with
  // 2048 tokens); the dX direction stays on this kernel (90 against 101 us)
  if (gp.M >= 192 && t256x128 >= 160)
    return TRANS ? gemm_launch<256, 128, TRANS>(gp, st) : launch_nf4_gemm_wide(gp, TRANS, 128, st);
  return gemm_launch<128, 128, TRANS>(gp, st);
}

}  // namespace

hipError_t launch_nf4_gemm(GemmParams &gp, bool trans, hipStream_t st) {
  return trans ? gemm_select<true>(gp, st) : gemm_select<false>(gp, st);
}

}  // namespace ql

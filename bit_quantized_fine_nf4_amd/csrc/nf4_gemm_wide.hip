// Fused NF4 dequant-GEMM, 256 x 256 tiles, for gfx950: the forward kernel
// below, and the dX kernel (nf4_gemm_wide_dx_kernel) further down.
//
// [MC] "1. NormalFloat" / [GO] "The core move": the 4-bit weights are
// dequantized to BF16 on the fly for the matrix multiplication and never stored
// in wider form.  C[M][N] = A[M][K] · B[K][N] with A = X and B[k][n] = W_hat[n][k]
// (codes row n, 64-weight blocks along k), plus the rank-r term s·T·L2 as extra
// K steps on the same accumulators ([MC] "The algebra", Eq. 3).
//
// Workgroup: 4 waves, one per SIMD.  Wave w owns output columns [64w, 64w + 64)
// of the tile and all 256 rows: 8 x 2 tiles of v_mfma_f32_32x32x16_bf16, 256
// accumulator registers.  Because no other wave needs its columns, each wave
// decodes its own B fragments straight into registers: lane (n, g) (n = lane % 32,
// g = lane / 32) loads the 16 code bytes of row n that hold k in [32g, 32g + 32)
// of the K step (one 64-weight block, so one scale), looks each byte up in a
// 256-entry LDS table of level pairs (level[high nibble], level[low nibble]),
// multiplies by the block's rebuilt scale a_hat and converts to bf16 pairs:
// MFMA group kk takes k = 32g + 8kk + 0..7, exactly the lane's bytes 4kk..4kk+3.
// B therefore never passes through LDS and needs no synchronisation.
// A (X, k-contiguous) is shared by all four waves: it goes from memory straight
// into a 4-stage LDS ring (buffer_load ... lds, 16 bytes per lane, 1 KB = 8 rows
// per instruction) between two and three K steps ahead, in unpadded 128-byte rows
// whose 16-byte chunks are XOR-swizzled by row so the fragment reads are free of
// bank conflicts.  One barrier per K step, placed after the step's third MFMA
// group rather than at its start: the last group's MFMAs then cover the reads of
// the next step's first A fragments and table entries, so a step no longer opens
// with an LDS round trip (2048 tokens, one MI355X: 314 -> 258 us on 8192 -> 8192,
// 826 -> 774 us on 8192 -> 22016, bit-identical results).
// Per K step and wave: 8 A-fragment reads per MFMA group, 64 MFMAs, 32 table
// reads and about 5 VALU operations per code byte for the next step's decode
// (issued between the current step's MFMA groups), 14 vector-memory operations
// (8 A copies, 2 code, 2 int8-scale, 2 second-level-scale loads), the B loads two
// steps ahead.

#include "gemm.h"

namespace ql {
namespace {

QL_DEV __amdgpu_buffer_rsrc_t wrsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}
QL_DEV u32x4 wload128(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}
QL_DEV f32x16 wmfma(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                0, 0);
}
typedef short s16x4w __attribute__((ext_vector_type(4)));
QL_DEV u32x4 wtr_pair(const uint16_t *lo, const uint16_t *hi) {
  typedef __attribute__((address_space(3))) s16x4w lds_s16x4;
  const s16x4w a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lo));
  const s16x4w b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(hi));
  const u32x2 ua = __builtin_bit_cast(u32x2, a), ub = __builtin_bit_cast(u32x2, b);
  return u32x4{ua[0], ua[1], ub[0], ub[1]};
}
// (a device function, not the builtin inline in a kernel template's lambda: there
// the host pass of this compiler drops the kernel's launch stub without a
// diagnostic, and loading the library then fails on the undefined symbol)
QL_DEV void wload16_to_lds(__amdgpu_buffer_rsrc_t r, uint16_t *dst, int voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}
QL_DEV uint16_t wbf16(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }
// Workgroup barrier without the memory fences of __syncthreads(): those make the
// compiler wait for every outstanding load, the prefetches included.  The K loop
// orders its LDS traffic itself (an explicit wait for this wave's own copies into
// LDS before the barrier); the empty asm statements keep the compiler from moving
// memory accesses across it.
QL_DEV void wbarrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Tiles are 256 x (128 TN): TN = 2 for 256-wide tiles, 1 for 128-wide ones.  Wave w
// owns output columns [32 TN w, 32 TN (w + 1)): TN tiles of 32 columns.
constexpr int kBM = 256, kBK = 64, kThreads = 256;
constexpr int kTM = 8;                // 32x32 MFMA tiles per wave along M
constexpr int kStageElems = kBM * kBK;  // 256 rows x 64 k (bf16)
constexpr int wmax(int a, int b) { return a > b ? a : b; }

// row r of an A stage keeps its 8 chunks of 16 bytes in the order c ^ swz(r)
QL_DEV int a_swz(int r) { return (r >> 1) & 7; }

}  // namespace

template <int TN>
__global__ __launch_bounds__(kThreads) void nf4_gemm_wide_fwd_kernel(GemmParams p) {
  constexpr int kTN = TN, kBN = 128 * TN, kWC = 32 * TN;
  // 256-wide tiles: a 3-stage A ring and a 64 KB pair table of 32 copies at a 256-byte
  // entry stride, so a lookup's address is one v_perm_b32 and every lane of a 32-lane
  // phase reads its own banks (41 fewer VALU instructions per step: the 65B block step
  // 7.81 -> 7.68 ms); 128-wide tiles keep a 4-stage ring and 16 copies at 128 bytes
  // (the 3-stage form measured 2 % slower there)
  constexpr bool kPermLut = TN == 2;
  constexpr int kStages = kPermLut ? 3 : 4;
  constexpr int kLutCopies = kPermLut ? 32 : 16;  // lane l reads copy l % kLutCopies
  constexpr int kLutStride = 8 * kLutCopies;       // bytes per table entry (level pair)
  constexpr int kLutBytes = 256 * kLutStride;
  constexpr int kLdc = kBN + 8;    // epilogue staging row stride (elements)
  constexpr int kLdkn = kBN + 32;  // LoRA B2 tile [64 k][kLdkn] (transposing reads)
  constexpr int kLdsBytes = wmax(kLutBytes + kStages * kStageElems * 2, kBM * kLdc * 2);
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  // kPermLut: the pair table at offset 0, so a lookup's address is one byte
  // permutation (the code byte above the lane's copy offset), the A ring after it;
  // otherwise the A ring first, so the fragment reads of all four buffers reach their
  // addresses from two base registers (16-bit offsets), the table after it
  char *const tab = kPermLut ? lds : lds + kStages * kStageElems * 2;
  uint16_t *ring = reinterpret_cast<uint16_t *>(kPermLut ? lds + kLutBytes : lds);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;

  for (int i = tid; i < 256 * kLutCopies; i += kThreads) {
    const int e = i / kLutCopies;  // word i at 8 i = entry e's stride + 8 x copy
    reinterpret_cast<f32x2 *>(tab)[i] = f32x2{p.level[e >> 4], p.level[e & 15]};
  }

  int tm, tn;
  gemm_tile_of(blockIdx.x, p.tiles_m, p.tiles_n, kTN == 2 ? 4 : 2, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int64_t mrows = p.M - m0 < kBM ? p.M - m0 : kBM;
  const int64_t nrows = p.N - n0 < kBN ? p.N - n0 : kBN;
  const float mu = *p.mean;
  const int64_t bpr = p.ldw >> 6;  // 64-blocks per codes row

  // ---- A: each wave copies 8 blocks of 8 rows per stage, lane L -> row 8 blk + L / 8,
  // physical chunk L % 8 (global chunk (L % 8) ^ swz(row))
  const auto rA = wrsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  // the swizzle of row 8 (8 wv + c) + lane / 8 depends on c only through c's parity,
  // so two lane offsets serve all eight copies; the rest of the row offset is uniform
  int voffA[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 8 * (wv * 8 + c) + (lane >> 3), lc = (lane & 7) ^ a_swz(r);
    voffA[c] = (int)((r * p.lda + lc * 8) * 2);
  }
  const int rowstepA = __builtin_amdgcn_readfirstlane((int)(8 * p.lda * 2));
  auto dma_a = [&](int kt_, int buf) {
    const int kt = __builtin_amdgcn_readfirstlane(kt_);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      wload16_to_lds(rA, ring + buf * kStageElems + (wv * 8 + c) * 8 * kBK, voffA[c & 1],
                     kt * kBK * 2 + (c & ~1) * rowstepA);
  };

  // ---- B: lane (l32, g) of wave w decodes codes rows 32 TN w + 32j + l32 (j < TN)
  const auto rC = wrsrc(p.codes + n0 * (p.ldw >> 1), nrows * (p.ldw >> 1));
  const auto rQ = wrsrc(p.qabsmax + n0 * bpr, nrows * bpr);
  const auto rS2 = wrsrc(p.scale2, ((p.wrows * bpr + 255) >> 8) * 4);
  int voffC[kTN], voffQ[kTN];
  int64_t blk0[kTN];
#pragma unroll
  for (int j = 0; j < kTN; ++j) {
    const int row = kWC * wv + 32 * j + l32;
    voffC[j] = (int)(row * (p.ldw >> 1) + 16 * g);
    voffQ[j] = (int)(row * bpr);
    blk0[j] = (n0 + row) * bpr;
  }
  struct BRegs {
    u32x4 c[kTN];     // 16 code bytes per row
    uint32_t q[kTN];  // int8 block scale, zero-extended
    float s2[kTN];    // its second-level step
  };
  auto load_b = [&](int kt_, BRegs &R) {
    const int kt = __builtin_amdgcn_readfirstlane(kt_);
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      R.c[j] = wload128(rC, voffC[j], kt * 32);
      R.q[j] = __builtin_amdgcn_raw_buffer_load_b8(rQ, voffQ[j], kt, 0);
      R.s2[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                              rS2, (int)(((blk0[j] + kt) >> 8) * 4), 0, 0));
    }
  };
  // kPermLut: lane l reads copy l % 32, so a 32-lane phase of 8-byte reads covers the
  // 64 banks once whatever the code bytes
  const int lcopy8 = (lane % kLutCopies) * 8;
  // Decode of one part (4 code bytes of each of the lane's two rows = MFMA group
  // `part`) in two halves so the table reads can run ahead of their use:
  //   lut_read: the 8 table reads (level pairs) of part `part`;
  //   lut_use:  the rebuilt scales times those levels, converted to bf16 pairs.
  typedef f32x2 Lv[kTN][4];
  auto lut_read = [&](const BRegs &R, int part, Lv &lv) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const uint32_t w = R.c[j][part];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if constexpr (kPermLut) {  // (byte b of w) << 8 | lcopy8
          const uint32_t addr = __builtin_amdgcn_perm(w, (uint32_t)lcopy8, 0x0C0C0000u | ((4u + b) << 8));
          lv[j][b] = *reinterpret_cast<const f32x2 *>(tab + addr);
        } else {
          const uint32_t byte = (w >> (8 * b)) & 0xFFu;
          lv[j][b] = *reinterpret_cast<const f32x2 *>(tab + (byte << 7) + lcopy8);
        }
      }
    }
  };
  auto scale_of = [&](const BRegs &R, float (&ah)[kTN]) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      // int8 from the zero-extended byte by float arithmetic (a sign-extending load
      // would be fused with the load and moved next to the younger prefetch)
      const float qf = (float)R.q[j] - (float)(R.q[j] & 0x80u) * 2.0f;
      ah[j] = qf * R.s2[j] + mu;  // two roundings: the library builds without contraction
    }
  };
  auto lut_use = [&](const Lv &lv, const float (&ah)[kTN], int part, u32x4 (&bf)[kTN][4]) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      uint32_t o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = pack_bf16x2(lv[j][b][0] * ah[j], lv[j][b][1] * ah[j]);
      bf[j][part] = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // A fragments of MFMA group kk from stage buffer `buf`: rows 32i + l32, chunk 4g + kk
  auto read_a = [&](int buf, int kk, u32x4 (&af)[kTM]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int r = 32 * i + l32;
      af[i] = *reinterpret_cast<const u32x4 *>(ring + buf * kStageElems + r * kBK + (((4 * g + kk) ^ a_swz(r)) << 3));
    }
  };

  // wait until at most n vector-memory operations of this wave are outstanding
  // (the LDS-bound A copies count; the compiler cannot know other waves read them)
  auto wait_vm = [](auto nconst) {
    constexpr int n = decltype(nconst)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
  };

  const int nk = p.ksteps;
  BRegs R0, R1;
  u32x4 bcur[kTN][4], bnext[kTN][4];
  u32x4 af[2][kTM];
  __syncthreads();  // pair table ready
  dma_a(0, 0);
  load_b(0, R0);
  __builtin_amdgcn_sched_barrier(0);
  dma_a(1, 1);
  load_b(1, R1);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kStages == 4) {
    dma_a(2, 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  {
    float ah[kTN];
    scale_of(R0, ah);
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      Lv lv;
      lut_read(R0, part, lv);
      lut_use(lv, ah, part, bcur);
    }
  }
  // step 0's B loads and so stage 0 are done once the younger operations (stage 1,
  // step 1's B loads and, with four stages, stage 2) are all that may be outstanding
  wait_vm(std::integral_constant<int, 8 * (kStages - 2) + 3 * TN>{});
  wbarrier();
  read_a(0, 0, af[0]);
  Lv lv[2];
  float ahn[kTN];
  lut_read(R1, 0, lv[0]);
  scale_of(R1, ahn);

  // Step kt (ring buffer BUF = kt % kStages, compile-time: the loop is unrolled six
  // (three stages) or four times; the two B register sets alternate).  On entry af[0] holds group 0's A
  // fragments of step kt, bcur its decoded B, lv[0] and ahn the first table reads
  // and scales of step kt + 1's decode.  Issued between group 0's MFMAs: the B
  // loads of step kt + 2 (into the set step kt's own B came from).  The decode of
  // step kt + 1 runs between the MFMAs: while group kk's MFMAs issue, the A
  // fragments of group kk + 1 and the table reads of part kk + 1 are in flight and
  // part kk's levels are scaled and converted.  After group 2's MFMAs this wave's
  // copy of stage kt + 1 is awaited, one barrier makes every wave's copy visible
  // and frees buffer (kt - 1) % kStages (last read in step kt - 1), and group 3
  // issues the copy of stage kt + kStages - 1 into it between its MFMAs, which also
  // cover the reads of step kt + 1's group-0 fragments and of the first part of step
  // kt + 2's decode.  Loads past the last step read harmless data that is never used.
  auto step = [&](auto bufc, int kt, BRegs &Rnext, BRegs &Rfree) {
    constexpr int BUF = decltype(bufc)::value;
    float ah[kTN];
#pragma unroll
    for (int j = 0; j < kTN; ++j) ah[j] = ahn[j];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) {
        if (kk == 0) load_b(kt + 2, Rfree);
        read_a(BUF, kk + 1, af[(kk + 1) & 1]);
        lut_read(Rnext, kk + 1, lv[(kk + 1) & 1]);
      } else {
        dma_a(kt + kStages - 1, (BUF + kStages - 1) % kStages);
        read_a((BUF + 1) % kStages, 0, af[0]);
        lut_read(Rfree, 0, lv[0]);
        scale_of(Rfree, ahn);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = wmfma(af[kk & 1][i], bcur[j][kk], acc[i][j]);
      lut_use(lv[kk & 1], ah, kk, bnext);
      // interleave: each MFMA followed by LDS reads and a few decode instructions
      // (128-wide tiles: half the MFMAs per group for the same A reads)
#pragma unroll
      for (int i = 0; i < 8 * TN; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);           // MFMA
        // the step's B loads ride on group 0, the copy of the next stage on group 3: issued
        // back to back by all four waves they queue at the compute unit's address unit
        // and stall the issuing wave, and the matrix core with it
        if ((kk == 0 && i < 3 * TN) || (kk == 3 && i < 8)) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
        __builtin_amdgcn_sched_group_barrier(0x100, TN == 2 ? 1 : 2, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, TN == 2 ? 2 : 3, 0);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 2) {
        // younger than this wave's copy of stage kt + 1: with three stages (issued in
        // step kt - 1's last group) the B loads of step kt + 2 (3 TN); with four the B
        // loads of step kt + 1, the copy of stage kt + 2 and the B loads of step kt + 2
        wait_vm(std::integral_constant<int, kStages == 3 ? 3 * TN : 8 + 6 * TN>{});
        wbarrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bcur[j][kk] = bnext[j][kk];
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  int kt = 0;
  if constexpr (kStages == 3) {
    for (; kt + 5 < nk; kt += 6) {
      step(I0{}, kt, R1, R0);
      step(I1{}, kt + 1, R0, R1);
      step(I2{}, kt + 2, R1, R0);
      step(I0{}, kt + 3, R0, R1);
      step(I1{}, kt + 4, R1, R0);
      step(I2{}, kt + 5, R0, R1);
    }
    if (kt < nk) step(I0{}, kt, R1, R0);
    if (kt + 1 < nk) step(I1{}, kt + 1, R0, R1);
    if (kt + 2 < nk) step(I2{}, kt + 2, R1, R0);
    if (kt + 3 < nk) step(I0{}, kt + 3, R0, R1);
    if (kt + 4 < nk) step(I1{}, kt + 4, R1, R0);
  } else {
    using I3 = std::integral_constant<int, 3>;
    for (; kt + 3 < nk; kt += 4) {
      step(I0{}, kt, R1, R0);
      step(I1{}, kt + 1, R0, R1);
      step(I2{}, kt + 2, R1, R0);
      step(I3{}, kt + 3, R0, R1);
    }
    if (kt < nk) step(I0{}, kt, R1, R0);
    if (kt + 1 < nk) step(I1{}, kt + 1, R0, R1);
    if (kt + 2 < nk) step(I2{}, kt + 2, R1, R0);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no copy of a stage past the end may still land in LDS
  __syncthreads();

  // ---- rank-r K steps: A2 = s-scaled T [M][lda2] through ring buffer 0, B2 = L2
  // [r][N] as a [k][n] tile (rows past r read as zero) in the space of buffers 1-2,
  // read with transposing loads (lane n receives column n's 8 consecutive k)
  if (p.ksteps2 > 0) {
    const auto rA2 = wrsrc(p.A2 + m0 * p.lda2, mrows * p.lda2 * 2);
    const auto rB2 = wrsrc(p.B2 + n0, ((int64_t)p.b2rows * p.ldb2 - n0) * 2);
    uint16_t *a2 = ring;
    uint16_t *b2 = ring + kStageElems;
    const int c = lane & 15;
    for (int k2 = 0; k2 < p.ksteps2; ++k2) {
      // A2: 256 rows x 64 k, 8 chunks per row (same swizzle as A), 8 per thread
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ch = tid + kThreads * u, r = ch >> 3, lc = ch & 7;
        const u32x4 v = wload128(rA2, (int)((r * p.lda2 + lc * 8) * 2), k2 * kBK * 2);
        *reinterpret_cast<u32x4 *>(a2 + r * kBK + ((lc ^ a_swz(r)) << 3)) = v;
      }
      // B2: 64 rows (k) x kBN columns, kBN / 8 chunks per row, kBN / 32 per thread
#pragma unroll
      for (int u = 0; u < kBN / 32; ++u) {
        const int ch = tid + kThreads * u, kr = (int)((unsigned)ch / (kBN / 8)), c8 = (int)((unsigned)ch % (kBN / 8));
        const u32x4 v = wload128(rB2, (int)(((int64_t)(k2 * kBK + kr) * p.ldb2 + c8 * 8) * 2), 0);
        *reinterpret_cast<u32x4 *>(b2 + kr * kLdkn + c8 * 8) = v;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 af[kTM];
        read_a(0, kk, af);
        u32x4 bf[kTN];
        const uint16_t *b0 = b2 + (32 * g + 8 * kk + (c >> 2)) * kLdkn + kWC * wv + ((lane >> 4) & 1) * 16 + (c & 3) * 4;
#pragma unroll
        for (int j = 0; j < kTN; ++j) bf[j] = wtr_pair(b0 + 32 * j, b0 + 4 * kLdkn + 32 * j);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) acc[i][j] = wmfma(af[i], bf[j], acc[i][j]);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: fp32 -> bf16 through LDS, then coalesced 16-byte stores
  uint16_t *cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        const int col = kWC * wv + 32 * j + l32;
        cs[row * kLdc + col] = wbf16(acc[i][j][v]);
      }
  __syncthreads();
  for (int ch = tid; ch < kBM * kBN / 8; ch += kThreads) {
    const int row = ch / (kBN / 8), c8 = ch % (kBN / 8);
    const int64_t m = m0 + row, n = n0 + c8 * 8;
    if (m < p.M && n < p.N)
      *reinterpret_cast<u32x4 *>(p.C + m * p.ldc + n) = *reinterpret_cast<const u32x4 *>(cs + row * kLdc + c8 * 8);
  }
}


// ---------------------------------------------------------------------------
// dX direction: C[M][N] = dY[M][K] · W_hat[K][N] + s·U·L1^T, K = o, N = h
// ([MC] "One training step": the gradient flows through the frozen dequantized
// weight).  Same four-wave split as the forward: wave w owns output columns
// [64w, 64w + 64) and all 256 rows, with 8 x 2 tiles of 32x32x16 MFMAs.  The
// stored codes run along N, so a wave's B fragment (8 consecutive k of one
// column) is a transpose of the stored rows:
//  - each K step's 64 code rows x 256 columns (8 KB) go to LDS by direct-to-LDS
//    loads, 16-byte chunks at chunk ^ ((row >> 1) & 7), in a 3-stage ring;
//  - one 4-bit transposing read (ds_read_b64_tr_b4) gives lane i of a 16-lane
//    group the nibbles of 16 consecutive rows of one column.  It returns a
//    byte's low nibble first, and a stored byte keeps the even column in its
//    high nibble, so lane i holds column i ^ 1: the epilogue (and the rank-r
//    operand) use the same swapped column, so every accumulator column is one
//    output column;
//  - each byte of the result is two consecutive rows of the column: one table
//    read gives both levels, each multiplied by its own row's a_hat (the block
//    scale belongs to a row and a 64-column block; a wave's 64 columns are one
//    block), then one packed conversion gives the MFMA dword;
//  - the 256 a_hat values of a stage (64 rows x the tile's 4 blocks) are
//    rebuilt by the 256 threads, one each, two steps ahead, and published in a
//    3-stage LDS ring; a lane reads its 8 values per MFMA group as two
//    broadcast 16-byte reads.
// A (dY) takes the forward's path, through a 2-stage ring: a stage's slot is free
// after the barrier of the step that reads it, which is where the copy two stages
// ahead is issued.  The pair table sits at offset 0 in 32 copies at a 256-byte
// entry stride: a lookup address is one v_perm_b32 of the code word and the lane's
// copy offset, and each lane of a 32-lane phase reads its own two banks.  With rings
// of two and three stages the K loop is unrolled six times, so every slot is a
// compile-time offset.  One barrier per K
// step after the third MFMA group, as in the forward; the last group's MFMAs
// cover the next step's first A fragments and the first part of the decode
// after next.
// ---------------------------------------------------------------------------
namespace {
constexpr int kXStagesA = 2;                  // A (dY) ring
constexpr int kXStages = 3;                   // code and a_hat rings
constexpr int kXBN = 256, kXTN = 2;           // 256-wide tiles: two 32-column MFMA tiles per wave
constexpr int kXLdc = kXBN + 8;               // epilogue staging row stride (elements)
constexpr int kXCodeBytes = 64 * (kXBN / 2);  // 64 code rows x 256 columns
constexpr int kXAhFloats = 4 * 64;            // [4 blocks][64 rows]
constexpr int kXLutCopies = 32;               // lane l reads copy l % 32 of the pair table
constexpr int kXLutStride = 8 * kXLutCopies;  // bytes per table entry: a lookup address is
                                              // (code byte) << 8 | 8 (lane % 32), one v_perm
constexpr int kXOffA = 256 * kXLutStride;     // the table at offset 0, then the rings
constexpr int kXOffC = kXOffA + kXStagesA * kStageElems * 2;
constexpr int kXOffS = kXOffC + kXStages * kXCodeBytes;
constexpr int kXLdsBytes = wmax(kXOffS + kXStages * kXAhFloats * 4, kBM * kXLdc * 2);
typedef int wi32x2 __attribute__((ext_vector_type(2)));
QL_DEV u32x2 wtr4(const uint8_t *ptr) {
  typedef __attribute__((address_space(3))) wi32x2 lds_i32x2;
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i32x2 *)(ptr)));
}
}  // namespace

__global__ __launch_bounds__(kThreads) void nf4_gemm_wide_dx_kernel(GemmParams p) {
  constexpr int kTN = kXTN, kBN = kXBN, kLdc = kXLdc;
  __shared__ __attribute__((aligned(16))) char lds[kXLdsBytes];
  char *const tab = lds;
  uint16_t *ring = reinterpret_cast<uint16_t *>(lds + kXOffA);
  uint8_t *cring = reinterpret_cast<uint8_t *>(lds + kXOffC);
  float *ahs = reinterpret_cast<float *>(lds + kXOffS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31, i16 = lane & 15, half = (lane >> 4) & 1;

  // entry e of copy c (at 256 e + 8 c): (level[low nibble], level[high nibble]), the
  // levels of a byte's earlier and later row
  for (int i = tid; i < 256 * kXLutCopies; i += kThreads) {
    const int e = i / kXLutCopies;
    reinterpret_cast<f32x2 *>(tab)[i] = f32x2{p.level[e & 15], p.level[e >> 4]};
  }

  int tm, tn;
  gemm_tile_of(blockIdx.x, p.tiles_m, p.tiles_n, 4, tm, tn);
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * kBN;
  const int64_t mrows = p.M - m0 < kBM ? p.M - m0 : kBM;
  const int64_t nrows = p.N - n0 < kBN ? p.N - n0 : kBN;
  const float mu = *p.mean;
  const int64_t bpr = p.ldw >> 6;   // 64-blocks per codes row
  const int64_t rowB = p.ldw >> 1;  // bytes per codes row

  // ---- A (dY): as in the forward, 8 copies of 8 rows per wave and stage
  const auto rA = wrsrc(p.A + m0 * p.lda, mrows * p.lda * 2);
  int voffA[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = 8 * (wv * 8 + c) + (lane >> 3), lc = (lane & 7) ^ a_swz(r);
    voffA[c] = (int)((r * p.lda + lc * 8) * 2);
  }
  const int rowstepA = __builtin_amdgcn_readfirstlane((int)(8 * p.lda * 2));
  auto dma_a = [&](int kt_, int buf) {
    const int kt = __builtin_amdgcn_readfirstlane(kt_);
#pragma unroll
    for (int c = 0; c < 8; ++c)
      wload16_to_lds(rA, ring + buf * kStageElems + (wv * 8 + c) * 8 * kBK, voffA[c & 1],
                     kt * kBK * 2 + (c & ~1) * rowstepA);
  };
  auto read_a = [&](int buf, int kk, u32x4 (&af)[kTM]) {
#pragma unroll
    for (int i = 0; i < kTM; ++i) {
      const int r = 32 * i + l32;
      af[i] = *reinterpret_cast<const u32x4 *>(ring + buf * kStageElems + r * kBK + (((4 * g + kk) ^ a_swz(r)) << 3));
    }
  };

  // ---- codes: wave w copies rows 8 (2w + j) + L / 8 (j = 0, 1) of a stage; lane L
  // fetches the logical chunk that belongs at physical chunk L % 8 of its row
  int voffC[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 8 * (2 * wv + j) + (lane >> 3), lc = (lane & 7) ^ a_swz(r);
    voffC[j] = (int)(r * rowB + 16 * lc);
  }
  auto dma_c = [&](int s_, int buf) {
    const int s = __builtin_amdgcn_readfirstlane(s_);
    const int64_t r0 = (int64_t)s * 64;
    const auto rC = wrsrc(p.codes + r0 * rowB + (n0 >> 1), (p.wrows - r0) * rowB - (n0 >> 1));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      wload16_to_lds(rC, reinterpret_cast<uint16_t *>(cring + buf * kXCodeBytes + 1024 * (2 * wv + j)), voffC[j], 0);
  };
  // transposing read t (rows 16t .. 16t + 15 of the lane's 32) of column tile j:
  // lane i of its 16-lane group names row 32 g + 16 t + i, whose swizzle is (i >> 1) & 7
  int troff[kTN];
#pragma unroll
  for (int j = 0; j < kTN; ++j) troff[j] = (32 * g + i16) * 128 + 16 * ((2 * wv + j) ^ ((i16 >> 1) & 7)) + 8 * half;
  auto read_tr = [&](int buf, int t, u32x2 (&tw)[kTN]) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) tw[j] = wtr4(cring + buf * kXCodeBytes + troff[j] + 16 * t * 128);
  };

  // ---- a_hat: thread t rebuilds row t / 4, block t % 4 of a stage
  const int qrow = tid >> 2, qblk = tid & 3;
  const auto rQ = wrsrc(p.qabsmax, p.wrows * bpr);
  const auto rS2 = wrsrc(p.scale2, ((p.wrows * bpr + 255) >> 8) * 4);
  struct QS {
    uint32_t q;  // int8 block scale, zero-extended
    float s2;
  };
  auto load_qs = [&](int s_, QS &Q) {
    const int s = __builtin_amdgcn_readfirstlane(s_);
    const int64_t bi = ((int64_t)s * 64 + qrow) * bpr + (n0 >> 6) + qblk;
    Q.q = __builtin_amdgcn_raw_buffer_load_b8(rQ, (int)bi, 0, 0);
    Q.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS2, (int)((bi >> 8) * 4), 0, 0));
  };
  auto put_ah = [&](const QS &Q, int buf) {
    // int8 from the zero-extended byte by float arithmetic; two roundings
    const float qf = (float)Q.q - (float)(Q.q & 0x80u) * 2.0f;
    ahs[buf * kXAhFloats + qblk * 64 + qrow] = qf * Q.s2 + mu;
  };

  // ---- decode of one part (MFMA group kk: rows 32 g + 8 kk .. + 7 of the lane's column)
  const int lcopy8 = (lane % kXLutCopies) * 8;
  typedef f32x2 XLv[kTN][4];
  auto lut_read = [&](const u32x2 (&tw)[kTN], int kk, XLv &lv) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      const uint32_t w = tw[j][kk & 1];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t addr = __builtin_amdgcn_perm(w, (uint32_t)lcopy8, 0x0C0C0000u | ((4u + d) << 8));
        lv[j][d] = *reinterpret_cast<const f32x2 *>(tab + addr);
      }
    }
  };
  auto sc_read = [&](int buf, int kk, f32x4 (&sc)[2]) {
    const float *sp = ahs + buf * kXAhFloats + wv * 64 + 32 * g + 8 * kk;
    sc[0] = *reinterpret_cast<const f32x4 *>(sp);
    sc[1] = *reinterpret_cast<const f32x4 *>(sp + 4);
  };
  auto lut_use = [&](const XLv &lv, const f32x4 (&sc)[2], int kk, u32x4 (&bf)[kTN][4]) {
#pragma unroll
    for (int j = 0; j < kTN; ++j) {
      uint32_t o[4];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = pack_bf16x2(lv[j][d][0] * sc[d >> 1][2 * (d & 1)], lv[j][d][1] * sc[d >> 1][2 * (d & 1) + 1]);
      bf[j][kk] = u32x4{o[0], o[1], o[2], o[3]};
    }
  };

  // lgkmcnt(0) (this wave's a_hat stores) and vmcnt(n) (its copies into LDS)
  auto wait_vm_lgkm = [](auto nconst) {
    constexpr int n = decltype(nconst)::value;
    __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | ((n >> 4) << 14));
  };

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = p.ksteps;
  // stage s lives in slot s % 2 of the A ring, slot s % 3 of the code and a_hat
  // rings, and its int8 / second-level scales in register set Qs[s % 3] until they
  // are published
  QS Qs[kXStages];
  u32x4 bcur[kTN][4], bnext[kTN][4];
  u32x4 af[2][kTM];
  XLv lv[2];
  f32x4 sc[2][2];
  u32x2 tw0[kTN], tw1[kTN];
  __syncthreads();  // pair table ready
  // Prologue: codes of stages 0-2, A of stages 0 and 1, the a_hat values of stages 0
  // and 1 published, the scales of stages 2 and 3 loaded; then stage 0 decoded, the
  // first reads of step 0 and of stage 1's decode, and, once every wave has read
  // stage 0's codes, the codes of stage 3 into their slot.
#pragma unroll
  for (int s = 0; s < 3; ++s) dma_c(s, s);
  dma_a(0, 0);
  load_qs(0, Qs[0]);
  load_qs(1, Qs[1]);
  __builtin_amdgcn_s_waitcnt(0);
  put_ah(Qs[0], 0);
  put_ah(Qs[1], 1);
  __builtin_amdgcn_sched_barrier(0);
  load_qs(2, Qs[2]);
  __builtin_amdgcn_sched_barrier(0);
  dma_a(1, 1);
  __builtin_amdgcn_sched_barrier(0);
  load_qs(3, Qs[0]);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();  // stage 0's A, stages 0-2's codes, a_hat of stages 0 and 1
  {
    read_tr(0, 0, tw0);
    read_tr(0, 1, tw1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      XLv l;
      f32x4 c2[2];
      lut_read(kk < 2 ? tw0 : tw1, kk, l);
      sc_read(0, kk, c2);
      lut_use(l, c2, kk, bcur);
    }
  }
  read_a(0, 0, af[0]);
  read_tr(1, 0, tw0);
  lut_read(tw0, 0, lv[0]);
  sc_read(1, 0, sc[0]);
  __syncthreads();  // every wave's reads of code slot 0 are done
  dma_c(3, 0);

  // Step kt (phase PH = kt % 6, compile-time: the loop is unrolled six times, so
  // every slot is a compile-time offset): A from slot kt % 2, B from bcur; decodes
  // stage kt + 1 into bnext (its part 0 read during step kt - 1).  On entry af[0]
  // holds group 0's A fragments, tw0 the first transposing reads of stage kt + 1,
  // lv[0] / sc[0] its part-0 table entries and scales.  At its start the a_hat values
  // of stage kt + 2 are published (slot (kt + 2) % 3, last read during step kt - 2).
  // After group 2: all of this wave's vector-memory operations (A stage kt + 1, code
  // stage kt + 3, the scales of stage kt + 3) and its a_hat stores are awaited, and
  // one barrier publishes every wave's copies and a_hat values and frees A slot
  // kt % 2 (stage kt, last read in group 2) and code slot (kt + 1) % 3 (stage kt + 1,
  // last read in group 0); group 3 then issues the copies of code stage kt + 4 and
  // A stage kt + 2 and the scale loads of stage kt + 4 between its MFMAs.  Copies and
  // loads past the last stage read harmless data (zero past the buffers' ends) that
  // is never used.
  auto step = [&](auto phc, int kt) {
    constexpr int PH = decltype(phc)::value;
    constexpr int BUF = PH % kXStagesA, BUF1 = (PH + 1) % kXStagesA;
    constexpr int B1 = (PH + 1) % kXStages, B2 = (PH + 2) % kXStages;
    put_ah(Qs[B2], B2);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk == 0) {
        read_a(BUF, 1, af[1]);
        read_tr(B1, 1, tw1);
        lut_read(tw0, 1, lv[1]);
        sc_read(B1, 1, sc[1]);
      } else if (kk == 1) {
        read_a(BUF, 2, af[0]);
        lut_read(tw1, 2, lv[0]);
        sc_read(B1, 2, sc[0]);
      } else if (kk == 2) {
        read_a(BUF, 3, af[1]);
        lut_read(tw1, 3, lv[1]);
        sc_read(B1, 3, sc[1]);
        read_tr(B2, 0, tw0);
      } else {
        dma_c(kt + 4, B1);
        dma_a(kt + 2, BUF);
        load_qs(kt + 4, Qs[B1]);
        read_a(BUF1, 0, af[0]);
        lut_read(tw0, 0, lv[0]);
        sc_read(B2, 0, sc[0]);
      }
#pragma unroll
      for (int i = 0; i < kTM; ++i)
#pragma unroll
        for (int j = 0; j < kTN; ++j) acc[i][j] = wmfma(af[kk & 1][i], bcur[j][kk], acc[i][j]);
      lut_use(lv[kk & 1], sc[kk & 1], kk, bnext);
      // interleave: each MFMA followed by one LDS read and three decode instructions
      // (two measured 2 % slower here: this decode has more VALU work per group); in
      // group 3 the first twelve also carry one of the step's twelve vector-memory
      // instructions (cycle stamps: issued back to back after the barrier, the four
      // waves' copies queued at the address unit for about 750 cycles)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                            // MFMA
        if (kk == 3 && i < 12) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                            // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);                            // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kk == 2) {
        // every vector-memory operation of the previous step (this wave's copies of A
        // stage kt + 1 and code stage kt + 3, the scale loads of stage kt + 3, issued
        // in group 3 in an order the scheduler chooses), this wave's a_hat stores, and
        // all of its LDS reads: with them done in every wave, the barrier frees the A
        // slot (stage kt, last read in group 2) and the code slot (stage kt + 1, last
        // read in group 0) that group 3's copies overwrite
        wait_vm_lgkm(std::integral_constant<int, 0>{});
        wbarrier();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) bcur[j][kk] = bnext[j][kk];
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  int kt = 0;
  for (; kt + 5 < nk; kt += 6) {
    step(I0{}, kt);
    step(I1{}, kt + 1);
    step(I2{}, kt + 2);
    step(I3{}, kt + 3);
    step(I4{}, kt + 4);
    step(I5{}, kt + 5);
  }
  if (kt < nk) step(I0{}, kt);
  if (kt + 1 < nk) step(I1{}, kt + 1);
  if (kt + 2 < nk) step(I2{}, kt + 2);
  if (kt + 3 < nk) step(I3{}, kt + 3);
  if (kt + 4 < nk) step(I4{}, kt + 4);
  __builtin_amdgcn_s_waitcnt(0);  // no copy of a stage past the end may still land in LDS
  __syncthreads();

  // ---- rank-r K steps: A2 = s-scaled U [M][lda2] through ring buffer 0; B2 = L1
  // padded to [N][ldb2]: lane (n, g) takes row n ^ 1 of its column tile (the
  // swapped column of the code path), 16 contiguous bytes per MFMA group
  if (p.ksteps2 > 0) {
    const auto rA2 = wrsrc(p.A2 + m0 * p.lda2, mrows * p.lda2 * 2);
    const auto rB2 = wrsrc(p.B2 + n0 * p.ldb2, nrows * p.ldb2 * 2);
    uint16_t *a2 = ring;
    for (int k2 = 0; k2 < p.ksteps2; ++k2) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ch = tid + kThreads * u, r = ch >> 3, lc = ch & 7;
        const u32x4 v = wload128(rA2, (int)((r * p.lda2 + lc * 8) * 2), k2 * kBK * 2);
        *reinterpret_cast<u32x4 *>(a2 + r * kBK + ((lc ^ a_swz(r)) << 3)) = v;
      }
      u32x4 b2[kTN][4];
#pragma unroll
      for (int j = 0; j < kTN; ++j)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          b2[j][kk] = wload128(rB2, (int)(((64 * wv + 32 * j + (l32 ^ 1)) * p.ldb2 + 32 * g + 8 * kk) * 2),
                               k2 * kBK * 2);
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 a[kTM];
        read_a(0, kk, a);
#pragma unroll
        for (int i = 0; i < kTM; ++i)
#pragma unroll
          for (int j = 0; j < kTN; ++j) acc[i][j] = wmfma(a[i], b2[j][kk], acc[i][j]);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: fp32 -> bf16 through LDS (accumulator column l32 is output column
  // l32 ^ 1 of its tile), then coalesced 16-byte stores
  uint16_t *cs = reinterpret_cast<uint16_t *>(lds);
#pragma unroll
  for (int i = 0; i < kTM; ++i)
#pragma unroll
    for (int j = 0; j < kTN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = 32 * i + 8 * (v >> 2) + 4 * g + (v & 3);
        const int col = 64 * wv + 32 * j + (l32 ^ 1);
        cs[row * kLdc + col] = wbf16(acc[i][j][v]);
      }
  __syncthreads();
  for (int ch = tid; ch < kBM * kBN / 8; ch += kThreads) {
    const int row = ch / (kBN / 8), c8 = ch % (kBN / 8);
    const int64_t m = m0 + row, n = n0 + c8 * 8;
    if (m < p.M && n < p.N)
      *reinterpret_cast<u32x4 *>(p.C + m * p.ldc + n) = *reinterpret_cast<const u32x4 *>(cs + row * kLdc + c8 * 8);
  }
}

hipError_t launch_nf4_gemm_wide(GemmParams &gp, bool trans, int bn, hipStream_t st) {
  if (bn != 256 && bn != 128) return hipErrorInvalidValue;
  gp.tiles_m = (int)((gp.M + kBM - 1) / kBM);
  gp.tiles_n = (int)((gp.N + bn - 1) / bn);
  const unsigned grid = (unsigned)(gp.tiles_m * gp.tiles_n);
  // the dX kernel has 256-wide tiles only: a 128-wide version measured slower than
  // the eight-wave kernel on a 4096 x 4096 weight with 2048 tokens (101 vs 90 us)
  if (trans) return bn == 256 ? launch(nf4_gemm_wide_dx_kernel, grid, kThreads, st, gp) : hipErrorInvalidValue;
  return bn == 256 ? launch(nf4_gemm_wide_fwd_kernel<2>, grid, kThreads, st, gp)
                   : launch(nf4_gemm_wide_fwd_kernel<1>, grid, kThreads, st, gp);
}

}  // namespace ql

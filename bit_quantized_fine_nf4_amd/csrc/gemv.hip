// Few-token NF4 forward for gfx950: Y = X·W_hat + s·T·L2 for M <= 16 tokens.
//
// [TT] §3 (the 4-bit storage) and [MC] "The algebra" (Eq. 3): with a handful
// of tokens the layer is one pass over the packed codes, read once from HBM.
// Two kernels:
//
// nf4_gemv1_kernel (one token).  Every wave walks a contiguous range of output
// features one whole row at a time, with 1 KB contiguous loads (64 lanes x 16
// bytes) eight loads ahead of use: long sequential runs per DRAM page, no
// cross-wave synchronisation, no staging of codes through LDS.  The token's
// activations for the whole K stay in registers (lane L holds the 32 weights of
// K it meets in each 1 KB load).  A code byte becomes its bf16 level pair through
// a 64-copy byte -> pair table in LDS (entry e of copy c at 256 e + 4 c; the
// address is one v_perm_b32 that puts the byte next to 4 x lane, and every lane
// reads its own bank), and v_dot2c_f32_bf16 multiplies the pair with the
// activation pair.  Each lane's 16 bytes are half of one 64-weight block, so the
// block scale a_hat multiplies the lane's partial sum.  At the end of a row the
// 64 lane sums meet by DPP and permlane swaps; the rank-r term is added per row.
//
// nf4_gemv_kernel (2 to 16 tokens).  A workgroup owns 64 output features and
// walks the whole K in stages of 256 weights (4 blocks): every stage (64 rows x
// 128 code bytes, 16 tokens x 512 activation bytes, 64 x 4 block scales) is
// fetched by all 512 threads with coalesced loads two stages ahead of use,
// parked in registers, then written to a double-buffered, XOR-swizzled LDS
// tile.  Wave w takes block w % 4 of every stage for row groups 2(w/4) and
// 2(w/4)+1 with 16x16x32 MFMAs, tokens being the MFMA rows.  The B operand is
// bf16(level[c]) from a byte -> bf16-pair table; a_hat multiplies each block's
// float32 partial.  The waves' partial sums meet in LDS at the end.

#include "gemv.h"

namespace ql {
namespace {

// Buffer resource over [base, base + bytes): loads past the end return zero.
QL_DEV __amdgpu_buffer_rsrc_t gv_rsrc(const void *base, int64_t bytes) {
  const int64_t cap = 0x7FFFFFF0;
  const int32_t n = (int32_t)(bytes < 0 ? 0 : (bytes > cap ? cap : bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, n, 0x00020000);
}

QL_DEV f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                0, 0);
}

QL_DEV uint16_t bf16_bits(float v) { return (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu); }

// ---------------------------------------------------------------------------
// One token
// ---------------------------------------------------------------------------
constexpr int kG1Threads = 256;   // 4 waves sharing the table
constexpr int kG1TargetWaves = 2048;  // two workgroups on each of the 256 compute units

template <int N>
QL_DEV float dpp_add(float x) {
  return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), N, 0xF, 0xF, false));
}

// sum over the 64 lanes, returned in every lane
QL_DEV float wave_sum(float x) {
  x = dpp_add<0xB1>(x);   // quad_perm 1 0 3 2
  x = dpp_add<0x4E>(x);   // quad_perm 2 3 0 1
  x = dpp_add<0x141>(x);  // row_half_mirror
  x = dpp_add<0x140>(x);  // row_mirror: each 16-lane row holds its sum
  // the four row sums, read from one lane of each row (wave-uniform result)
  const int xi = __builtin_bit_cast(int, x);
  return (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16))) +
         (__builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32)) +
          __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48)));
}

struct G1Load {
  u32x4 c;     // 16 code bytes: 32 weights, half of one block
  uint32_t q;  // that block's int8 scale, zero-extended
  float s2;    // its second-level scale
};

}  // namespace

// P: 1 KB loads per row whose activations are held in registers (K <= 2048 P).
template <int P>
__global__ __launch_bounds__(kG1Threads) __attribute__((amdgpu_waves_per_eu(2, 4))) void nf4_gemv1_kernel(
    GemvParams p, int rows_per_wave) {
  // one row of loads in flight: deeper rings measured slower (K = 8192: one, two and
  // four rows ahead took 26.0, 27.6 and 31.1 us), as more rows open at once cost
  // DRAM page locality; a ring of P also starts every pass on a row boundary
  constexpr int kG1Ring = P;
  __shared__ __attribute__((aligned(1024))) uint8_t lut[256 * 256];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  {
    // entry e = tid of every copy: bf16 pair (level[e >> 4], level[e & 15]) (a
    // byte's first weight sits in its high nibble and in the low half of the pair)
    const uint32_t pair = pack_bf16x2(p.level[tid >> 4], p.level[tid & 15]);
    const u32x4 p4 = {pair, pair, pair, pair};
#pragma unroll
    for (int c = 0; c < 64; c += 4) *reinterpret_cast<u32x4 *>(lut + tid * 256 + 4 * c) = p4;
  }
  // activations: xr[j][e] = X[0][2048 j + 32 lane + 8 e .. + 8) (zero past K)
  const __amdgpu_buffer_rsrc_t rx = gv_rsrc(p.X, p.K * 2);
  u32x4 xr[P][4];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int k0 = 2048 * j + 32 * lane + 8 * e;
      xr[j][e] = __builtin_amdgcn_raw_buffer_load_b128(rx, k0 < p.K ? 2 * k0 : (int)0x80000000, 0, 0);
    }
  __syncthreads();  // table ready

  const int64_t r0 = ((int64_t)blockIdx.x * 4 + wave) * rows_per_wave;
  const int64_t r1 = r0 + rows_per_wave < p.N ? r0 + rows_per_wave : p.N;
  const int nrows = r0 < r1 ? (int)(r1 - r0) : 0;
  const int64_t rowB = p.K >> 1, nblk = p.K >> 6;
  const __amdgpu_buffer_rsrc_t rc = gv_rsrc(p.codes + r0 * rowB, nrows * rowB);
  const __amdgpu_buffer_rsrc_t rq = gv_rsrc(p.qabsmax + r0 * nblk, nrows * nblk);
  const __amdgpu_buffer_rsrc_t rs = gv_rsrc(p.scale2, ((p.N * nblk + kChunk - 1) / kChunk) * 4);
  const float mu = *p.mean;
  const uint32_t lane4 = 4u * (uint32_t)lane;
  const int total = nrows * P;  // 1 KB loads of this wave

  // load i: row i / P, bytes [1024 (i % P) + 16 lane, + 16) of it (block 32 (i % P) + lane / 2).
  // 32-bit offsets and selects only (no branch), so the loaded registers carry
  // straight around the loop.
  const int rowBi = (int)rowB, nblki = (int)nblk;
  const int sfirst = (int)(r0 * nblk);  // flattened index of the wave's first block scale
  auto issue = [&](G1Load &L, int i) {
    const int rl = i / P, j = i % P;
    const int cb = 1024 * j + 16 * lane;
    const int blk = 32 * j + (lane >> 1);
    const bool in = i < total && cb < rowBi;
    const int oc = in ? rl * rowBi + cb : (int)0x80000000;
    const int oq = in ? rl * nblki + blk : (int)0x80000000;
    const int os = in ? ((sfirst + rl * nblki + blk) >> 8) << 2 : (int)0x80000000;
    // the codes are read once: non-temporal (cache policy NT; 8192 x 28672 weight under
    // a kernel trace 28.9 -> 25.2 us; the 4- and 16-token kernel and the few-token dX
    // measured no faster with it)
    L.c = __builtin_amdgcn_raw_buffer_load_b128(rc, oc, 0, 2);
    L.q = __builtin_amdgcn_raw_buffer_load_b8(rq, oq, 0, 0);
    L.s2 = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, os, 0, 0));
  };
  auto dot16 = [&](const G1Load &L, const u32x4 (&x)[4]) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t w = L.c[e];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // byte 1 of the address = byte t of w, byte 0 = 4 x lane
        const uint32_t a = __builtin_amdgcn_perm(w, lane4, 0x0C0C0000u | ((4u + t) << 8));
        const uint32_t lv = *reinterpret_cast<const uint32_t *>(lut + a);
        // the element goes through a scalar first: a bit cast applied directly to a
        // vector element reads element 0 with this compiler
        const uint32_t xv = x[e][t];
        if (t & 1)
          s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lv), __builtin_bit_cast(bf16x2, xv), s1, false);
        else
          s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, lv), __builtin_bit_cast(bf16x2, xv), s0, false);
      }
    }
    return s0 + s1;
  };

  G1Load ring[kG1Ring];
  // one load at a time, in the loop's own order, so the wait counts the compiler
  // derives for the ring are the same on entry as around the loop
#pragma unroll
  for (int d = 0; d < kG1Ring; ++d) {
    issue(ring[d], d);
    __builtin_amdgcn_sched_barrier(0);
  }
  float acc = 0.0f, ymine = 0.0f;  // ymine: total of row `lane` of this wave
  for (int i0 = 0; i0 < total; i0 += kG1Ring) {
#pragma unroll
    for (int d = 0; d < kG1Ring; ++d) {
      const int j = d % P;  // the ring and the row both line up with i0
      const float part = dot16(ring[d], xr[j]);
      // int8 from the zero-extended byte by float arithmetic; a_hat with two roundings
      const float qf = (float)ring[d].q - (float)(ring[d].q & 0x80u) * 2.0f;
      const float ah = qf * ring[d].s2 + mu;
      __builtin_amdgcn_sched_barrier(0);
      issue(ring[d], i0 + d + kG1Ring);
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_fmaf(ah, part, acc);
      if (j == P - 1) {
        const float tot = wave_sum(acc);
        const int rl = (i0 + d) / P;
        if (lane == (rl & 63)) ymine = tot;
        acc = 0.0f;
        if ((rl & 63) == 63 || rl == nrows - 1) {
          // flush up to 64 finished rows: the rank-r term, then one coalesced store
          const int first = rl & ~63;
          if (first + lane <= rl) {
            const int64_t col = r0 + first + lane;
            float y = ymine;
            for (int q = 0; q < p.r; ++q) y = __builtin_fmaf(bf16_lo(p.sT[q]), bf16_lo(p.L2[(int64_t)q * p.N + col]), y);
            p.Y[col] = bf16_bits(y);
          }
        }
      }
    }
  }
}

namespace {
// ---------------------------------------------------------------------------
// 2 to 16 tokens
// ---------------------------------------------------------------------------
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


}  // namespace

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
    p.Y[(int64_t)m * p.ldy + col] = bf16_bits(y);
  }
}

namespace {

}  // namespace

hipError_t launch_nf4_gemv(const GemvParams &p, hipStream_t st) {
  if (p.M == 1 && p.K <= 16384) {
    const int64_t per = (p.N + kG1TargetWaves - 1) / kG1TargetWaves;
    const int rows = (int)(per < 1 ? 1 : per);
    const unsigned grid = (unsigned)((p.N + 4 * (int64_t)rows - 1) / (4 * (int64_t)rows));
    return p.K <= 8192 ? launch(nf4_gemv1_kernel<4>, grid, kG1Threads, st, p, rows)
                       : launch(nf4_gemv1_kernel<8>, grid, kG1Threads, st, p, rows);
  }
  const unsigned grid = (unsigned)(p.N / kGvRows);
  auto k = p.M == 1 ? nf4_gemv_kernel<1> : (p.M <= 4 ? nf4_gemv_kernel<4> : nf4_gemv_kernel<16>);
  return launch(k, grid, kGvThreads, st, p);
}

}  // namespace ql

// NF4 codec kernels for gfx950: blockwise quantization, double quantization
// of the block scales, dequantization.  All bandwidth-bound: every kernel
// streams its inputs once with 16-byte loads and writes its outputs once with
// coalesced stores.  Compiled with -ffp-contract=off so that every float32
// operation written below rounds separately, as the method's steps state.

#include "codec.h"

#include <mutex>
#include <type_traits>
#include <vector>

namespace ql {

// ---------------------------------------------------------------------------
// Blockwise NF4 quantization ([MC] "1. NormalFloat"; [TT] §2 "Choose a scale,
// then round", §3; blocks of 64: [MC] "2. Double quantization").
//
// Lane layout: each lane owns 8 consecutive weights, so the 8 lanes of a
// half-row own one 64-weight block.  The block's largest magnitude is reduced
// with three DPP max steps inside the 8-lane group.  Each weight's code comes
// from the bucket table (see nf4_tables.hip): y = fma(w, 16/absmax, yoff),
// bucket floor(y), one comparison against the bucket's guard band.  A weight
// inside a guard band is decided by the IEEE division against the one
// threshold there; a block whose scale is 0 or outside [2^-100, 2^100] takes
// the IEEE division for all its codes.  The 8 codes
// are packed into one 32-bit word (first weight in the high nibble of the
// first byte) and stored with one coalesced dword store per lane.
// ---------------------------------------------------------------------------

QL_DEV float dpp_max8(float v) {
  // xor 1 and xor 2 inside each quad, then mirror inside the 8-lane half-row.
  int x = __builtin_bit_cast(int, v);
  float t = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  v = fmaxf(v, t);
  x = __builtin_bit_cast(int, v);
  t = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  v = fmaxf(v, t);
  x = __builtin_bit_cast(int, v);
  t = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false));
  return fmaxf(v, t);
}

// The weights are read once: non-temporal loads keep them from displacing what the
// caches hold (one LLaMA-65B block's seven float32 weights: quantize 118 -> 109 us
// per linear, and the dequantization that follows it 48 -> 45 us with its stores
// non-temporal as well).
template <bool kBf16>
QL_DEV void load8(const void *w, int64_t e0, int64_t n, float v[8]) {
  if (e0 + 8 <= n) {
    if (kBf16) {
      u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(w) + e0));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(d[i]);
        v[2 * i + 1] = bf16_hi(d[i]);
      }
    } else {
      const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(w) + e0);
      f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = a[i];
        v[4 + i] = b[i];
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t e = e0 + i;
      float x = 0.0f;
      if (e < n) {
        if (kBf16) x = __builtin_bit_cast(float, (uint32_t)reinterpret_cast<const uint16_t *>(w)[e] << 16);
        else x = reinterpret_cast<const float *>(w)[e];
      }
      v[i] = x;
    }
  }
}

QL_DEV uint32_t exact_code(float x, const Nf4Tables &t) {
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (x > t.thr[j]) ? 1u : 0u;
  return c;
}

// Codes of 8 consecutive weights of one block whose largest magnitude is a
// (already reduced over the block): element i in byte i/2, even i in the high
// nibble.  Fast path: y = 16 * x + yoff indexes a bucket of the threshold
// table.  A weight whose y falls inside its bucket's guard band is decided by
// the exact rule for the one threshold that can matter there: x = fp32(w / a)
// (IEEE division) against the bucket's float32 threshold tx.  A scale outside
// [2^-100, 2^100] takes the exact divide-and-compare path for all 8 weights.
// Either way the result equals the nearest-level rule on fp32(w / a).
QL_DEV uint32_t encode8(const float (&v)[8], float a, const EncBucket *lut, const Nf4Tables &tab) {
  uint32_t word = 0;
  if (a >= 0x1p-100f && a <= 0x1p100f) {
    const float r16 = 16.0f * __builtin_amdgcn_rcpf(a);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y = __builtin_fmaf(v[i], r16, tab.yoff);
      uint32_t idx = (uint32_t)(int32_t)y;
      idx = idx > (uint32_t)(kBuckets - 1) ? (uint32_t)(kBuckets - 1) : idx;
      const EncBucket e = lut[idx];
      const bool up = y > e.hi;
      uint32_t c = e.base + (up ? 1u : 0u);
      if ((y > e.lo) && !up) c = e.base + ((v[i] / a > e.tx) ? 1u : 0u);
      word |= c << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = a > 0.0f ? v[i] / a : 0.0f;
      word |= exact_code(x, tab) << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
    }
  }
  return word;
}

QL_DEV float absmax8(const float (&v)[8]) {
  return fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
               fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
}

template <bool kBf16>
__global__ __launch_bounds__(256) void quantize_kernel(const void *__restrict__ w, int64_t n,
                                                       uint8_t *__restrict__ codes,
                                                       float *__restrict__ absmax, Nf4Tables tab) {
  __shared__ EncBucket lut[kBuckets];
  if (threadIdx.x < kBuckets) lut[threadIdx.x] = tab.bucket[threadIdx.x];
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / 64);
  const int64_t ncodes = (n + 1) >> 1;

  auto encode = [&](const float (&v)[8], int64_t e0) {
    const float a = dpp_max8(absmax8(v));
    uint32_t word = encode8(v, a, lut, tab);
    const int64_t c0 = e0 >> 1;  // first byte index of this lane
    if (e0 + 8 <= n) {
      *reinterpret_cast<uint32_t *>(codes + c0) = word;
    } else if (e0 < n) {
      // tail: pad codes beyond n are the zero level's code, bytes beyond ceil(n/2) untouched
      for (int i = 0; i < 8; ++i)
        if (e0 + i >= n) word = (word & ~(0xFu << (8 * (i >> 1) + ((i & 1) ? 0 : 4)))) |
                                (tab.zero_code << (8 * (i >> 1) + ((i & 1) ? 0 : 4)));
      for (int b = 0; b < 4; ++b)
        if (c0 + b < ncodes) codes[c0 + b] = (uint8_t)(word >> (8 * b));
    }
    if ((lane & 7) == 0 && e0 < n) absmax[e0 >> 6] = a;
  };

  // Two 512-weight chunks per wave iteration, both loads issued before either is encoded.
  const int64_t stride = nwaves * 512;
  for (int64_t base = wave * 512; base < n; base += 2 * stride) {
    const int64_t e0 = base + lane * 8, e1 = base + stride + lane * 8;
    float v0[8], v1[8];
    load8<kBf16>(w, e0, n, v0);
    load8<kBf16>(w, e1, n, v1);
    encode(v0, e0);
    if (base + stride < n) encode(v1, e1);
  }
}

// ---------------------------------------------------------------------------
// Adapter merge ([TT] §11 "Saving, Loading, and Merging QLoRA Adapters"): the
// base is dequantized to a wider precision, the LoRA update added, and the
// result optionally quantized again.  Stored [o][h] entry (n, k) of
//   W' = W_hat + s * L1·L2            (W_hat h x o, L1 h x r, L2 r x o)
// is fp32(w_hat + fp32(s * P)) with w_hat = fp32(level * a_hat) exactly as
// qlora_dequantize computes it and P = sum_q L1[k][q] * L2[q][n] from bf16
// MFMAs with float32 accumulation.
//
// A workgroup owns a strip of 64 rows n and walks a range of 64-column k
// tiles (one quantization block of every row per tile).  Wave w owns rows
// 16w..16w+15: its MFMA B operand (L2 transposed, 16 rows x r) is built once
// in LDS and then held in registers.  Per tile, the 64 x r slice of L1
// (contiguous in memory) goes through a double-buffered LDS tile as the A
// operand shared by the four waves, and the A rows are permuted so that lane
// (i, g) ends up holding P for row 16w + i at the 16 consecutive columns
// 16g..16g+15: the 16x16x32 MFMA accumulators feed the epilogue directly.
// The strip's codes and rebuilt block scales come through LDS in chunks of
// kMergeChunk tiles (one contiguous run per row: short per-row reads spread
// over many rows cost HBM efficiency).  Each lane decodes its 16 codes, adds
// s * P, and stores 16 weights (fp32 / bf16), or re-encodes them with the
// encoder of qlora_quantize (block absmax over the row's 4 lanes, nearest
// level, packed codes).  One barrier per tile.
// ---------------------------------------------------------------------------
struct MergeParams {
  const uint8_t *codes;
  const int8_t *qabsmax;
  const float *scale2;
  const float *mean;
  int64_t h, o;
  const uint16_t *L1;  // [h][r]
  const uint16_t *L2;  // [r][o]
  int r;
  float s;
  int kper;             // k tiles per workgroup
  void *out;            // modes 0 / 1: [o][h] float32 / bf16
  uint8_t *codes_out;   // mode 2
  float *absmax_out;    // mode 2
};

constexpr int kMergeChunk = 4;                    // tiles per staged chunk of codes
constexpr int kMergeRowBytes = kMergeChunk * 32;  // code bytes per row per chunk

QL_DEV f32x4 mfma16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// MODE 0: float32 W'; 1: bf16 W'; 2: NF4 codes + absmax of W'.  RQ = ceil(r / 32) (0: no adapter).
template <int MODE, int RQ>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p, Nf4Tables tab) {
  constexpr int RP = 32 * (RQ > 0 ? RQ : 1);
  // LDS tile: row k holds q = 0..RP-1 with its 16-byte pieces permuted, piece c stored at
  // c ^ swz(k).  The MFMA A reads of one 16-lane pass take rows {a + 16 b + 4 t : a, b < 4}
  // and one piece each; the permutation puts those 16 reads on 16 distinct 4-bank groups
  // (for RP = 96 the 48-bank row stride alone does).
  constexpr int LDR = RP;
  constexpr int TILE = RQ > 0 ? 64 * LDR : 8;  // one buffer
  auto swz = [](int k) {
    return RP == 32 ? (k >> 4) & 3
         : RP == 64 ? ((k >> 1) & 1) | (((k >> 4) & 3) << 1)
         : RP == 128 ? (k & 3) | (((k >> 4) & 3) << 2) : 0;
  };
  auto radr = [&](int k, int q) { return k * LDR + 8 * ((q >> 3) ^ swz(k)) + (q & 7); };
  __shared__ __attribute__((aligned(16))) uint16_t tile[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint8_t cbuf[2][64][kMergeRowBytes + 16];  // codes
  __shared__ float abuf[2][64][kMergeChunk + 1];                                      // a_hat
  __shared__ f32x2 lv2[256];
  __shared__ EncBucket lut[kBuckets];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i = lane & 15, g = lane >> 4;
  lv2[tid] = f32x2{tab.level[tid >> 4], tab.level[tid & 15]};
  if (MODE == 2 && tid < kBuckets) lut[tid] = tab.bucket[tid];

  const int64_t h = p.h, nblk = h >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t row = n0 + 16 * wave + i;
  const int ta = (int)blockIdx.y * p.kper;
  const int tb = (int)(ta + p.kper < nblk ? ta + p.kper : nblk);
  const int r = p.r;
  const float mu = *p.mean;

  // Chunk staging: thread t copies bytes [32 (t & 3), +32) of row t >> 2's chunk of codes
  // (clamped into the valid part of a short last chunk), and rebuilds a_hat for the
  // (row, tile) pair t of the chunk.
  static_assert(kMergeRowBytes == 4 * 32 && 64 * kMergeChunk == 256, "staging split");
  struct Stage {
    u32x4 c[2];
    int qa;
    float s2;
  };
  auto stage_load = [&](int c0, Stage &st) {
    const int nt = tb - c0 < kMergeChunk ? tb - c0 : kMergeChunk;
    const uint8_t *base = p.codes + (((n0 + (tid >> 2)) * h + (int64_t)c0 * 64) >> 1);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      int off = 32 * (tid & 3) + 16 * u;
      off = off < 32 * nt - 16 ? off : 32 * nt - 16;
      st.c[u] = *reinterpret_cast<const u32x4 *>(base + off);
    }
    int tt = tid % kMergeChunk;
    tt = tt < nt ? tt : nt - 1;
    const int64_t blk = (n0 + tid / kMergeChunk) * nblk + c0 + tt;
    st.qa = p.qabsmax[blk];
    st.s2 = p.scale2[blk / kChunk];
  };
  auto stage_store = [&](int buf, const Stage &st) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *reinterpret_cast<u32x4 *>(&cbuf[buf][tid >> 2][32 * (tid & 3) + 16 * u]) = st.c[u];
    abuf[buf][tid / kMergeChunk][tid % kMergeChunk] = scale_hat((int8_t)st.qa, st.s2, mu);
  };

  // L1 slice of tile kt: 64 rows x r bf16 contiguous, 8r pieces of 16 bytes;
  // thread tid takes pieces tid + 256 m (clamped: surplus lanes reload the last piece).
  u32x4 lr[RQ > 0 ? RQ : 1];
  const int npc = 8 * r;
  auto load_l1 = [&](int kt) {
    const uint16_t *base = p.L1 + (int64_t)kt * 64 * r;
#pragma unroll
    for (int m = 0; m < RQ; ++m) {
      int c = tid + 256 * m;
      c = c < npc ? c : npc - 1;
      lr[m] = *reinterpret_cast<const u32x4 *>(base + 8 * c);
    }
  };
  int soff[RQ > 0 ? RQ : 1];  // LDS offset of each piece when r is a multiple of 8
#pragma unroll
  for (int m = 0; m < RQ; ++m) {
    const int c = tid + 256 * m, k = (8 * c) / r;
    soff[m] = radr(k, 8 * c - k * r);
  }
  auto store_l1 = [&](uint16_t *buf) {
#pragma unroll
    for (int m = 0; m < RQ; ++m) {
      const int c = tid + 256 * m;
      if (c < npc) {
        if ((r & 7) == 0) {
          *reinterpret_cast<u32x4 *>(&buf[soff[m]]) = lr[m];
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int e = 8 * c + j, k = e / r, q = e - k * r;
            buf[radr(k, q)] = (uint16_t)(lr[m][j >> 1] >> (16 * (j & 1)));
          }
        }
      }
    }
  };

  u32x4 bfr[RQ > 0 ? RQ : 1];
  if (RQ > 0) {
    // zero the padding columns q in [r, RP) of both buffers; stage L2^T of the strip in buffer 1
    for (int idx = tid; idx < 2 * 64 * (RP - r); idx += 256) {
      const int row2 = idx / (RP - r), q = r + idx % (RP - r);
      tile[(row2 >> 6) * TILE + radr(row2 & 63, q)] = 0;
    }
    for (int c = tid; c < npc; c += 256) {
      const int q = c >> 3, cn = c & 7;
      const u32x4 d = *reinterpret_cast<const u32x4 *>(p.L2 + (int64_t)q * p.o + n0 + 8 * cn);
#pragma unroll
      for (int j = 0; j < 8; ++j) tile[TILE + radr(8 * cn + j, q)] = (uint16_t)(d[j >> 1] >> (16 * (j & 1)));
    }
  }
  Stage st;
  stage_load(ta, st);
  if (RQ > 0) load_l1(ta);
  stage_store(0, st);
  __syncthreads();
  if (RQ > 0) {
#pragma unroll
    for (int qq = 0; qq < RQ; ++qq)
      bfr[qq] = *reinterpret_cast<const u32x4 *>(&tile[TILE + radr(16 * wave + i, 32 * qq + 8 * g)]);
    store_l1(tile);
  }
  __syncthreads();

  // One tile: its L1 slice is in LDS tile buffer `tbuf`, its codes in chunk buffer `cb`
  // at tile offset `ct`.
  auto step = [&](const int kt, const int tbuf, const int cb, const int ct) {
    if (RQ > 0) load_l1(kt + 1 < tb ? kt + 1 : kt);
    const u32x2 cw = *reinterpret_cast<const u32x2 *>(&cbuf[cb][16 * wave + i][32 * ct + 8 * g]);
    const float ah = abuf[cb][16 * wave + i][ct];
    float v[16];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const f32x2 l = lv2[(cw[b >> 2] >> (8 * (b & 3))) & 0xFF];
      v[2 * b] = l[0] * ah;
      v[2 * b + 1] = l[1] * ah;
    }
    if (RQ > 0) {
      const uint16_t *buf = tile + tbuf * TILE;
      // tile t, A row m = i -> column 16 (i >> 2) + 4 t + (i & 3); lane (i, g) receives
      // P at columns 16 g + 4 t + v, v = 0..3, of row 16 wave + i
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const int ka = 16 * (i >> 2) + 4 * t + (i & 3);
#pragma unroll
        for (int qq = 0; qq < RQ; ++qq) {
          const u32x4 a = *reinterpret_cast<const u32x4 *>(&buf[radr(ka, 32 * qq + 8 * g)]);
          acc = mfma16x32(a, bfr[qq], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float tt = p.s * acc[e];
          v[4 * t + e] = v[4 * t + e] + tt;
        }
      }
    }
    const int64_t e0 = row * h + (int64_t)kt * 64 + 16 * g;
    if (MODE == 0) {
      f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + e0);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) o[q4] = f32x4{v[4 * q4], v[4 * q4 + 1], v[4 * q4 + 2], v[4 * q4 + 3]};
    } else if (MODE == 1) {
      u32x4 *o = reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(p.out) + e0);
      o[0] = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7])};
      o[1] = u32x4{pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]), pack_bf16x2(v[12], v[13]),
                   pack_bf16x2(v[14], v[15])};
    } else {
      const float (&v0)[8] = *reinterpret_cast<const float (*)[8]>(&v[0]);
      const float (&v1)[8] = *reinterpret_cast<const float (*)[8]>(&v[8]);
      float a = fmaxf(absmax8(v0), absmax8(v1));
      a = fmaxf(a, __shfl_xor(a, 16));
      a = fmaxf(a, __shfl_xor(a, 32));
      *reinterpret_cast<u32x2 *>(p.codes_out + (e0 >> 1)) = u32x2{encode8(v0, a, lut, tab), encode8(v1, a, lut, tab)};
      p.absmax_out[row * nblk + kt] = a;  // the row's 4 lanes store the same value (no branch)
    }
    if (RQ > 0) store_l1(tile + (1 - tbuf) * TILE);
  };

  int j = 0;
  for (int c0 = ta; c0 < tb; c0 += kMergeChunk) {
    const int cb = ((c0 - ta) / kMergeChunk) & 1;
    const int ce = c0 + kMergeChunk < tb ? c0 + kMergeChunk : tb;
    const bool more = ce < tb;
    if (more) stage_load(ce, st);
    for (int kt = c0; kt < ce; ++kt, ++j) {
      step(kt, j & 1, cb, kt - c0);
      if (more && kt + 1 == ce) stage_store(cb ^ 1, st);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// Double quantization ([MC] "2. Double quantization"; [TT] §6 and §2's
// symmetric int8 scheme).
//
// The mean of the block scales is computed exactly: every float32 is an
// integer multiple of 2^-149, so their sum is an integer, accumulated without
// rounding and rounded once at the very end.  Two launches, with no
// cross-workgroup counter and nothing to clear beforehand:
//  dq_partial_kernel  each workgroup sums its share of the scales exactly and
//                     writes that integer as kLimbs 64-bit limbs (limb j holds
//                     bits [32j, 32j + 32), unnormalised, so it may exceed
//                     2^32) into its own slot of the workspace.  Inside the
//                     workgroup each lane keeps a 64-bit accumulator for an
//                     8-exponent window anchored at its first nonzero value;
//                     a value outside the window goes to its LDS exponent bin.
//  dq_chunks_kernel   every workgroup issues the loads of its first chunks'
//                     scales, adds the limbs of all slots, carries, divides by
//                     the count with correct rounding (mean_from_limbs) and
//                     quantizes its chunks; workgroup 0 also stores the mean.
//                     Integer addition is exact, so every workgroup derives
//                     the same mean whatever the order of the additions.
// ---------------------------------------------------------------------------

constexpr int kNumBins = 264;  // bin s holds integers in units of 2^(s-149)
constexpr int kDqGrid = 512;   // workgroups of the partial-sum pass (at most)
constexpr int kDqChGrid = 1024;  // workgroups of the chunk pass (at most; they loop)
constexpr int kLimbs = 12;     // the exact sum is below 2^(64+263): 11 32-bit limbs suffice

QL_DEV void split_f32(float a, uint32_t &mant, int &shift) {
  uint32_t b = __builtin_bit_cast(uint32_t, a);
  uint32_t e = (b >> 23) & 0xFF;
  mant = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  shift = e ? (int)e - 1 : 0;  // value = mant * 2^(shift - 149)
}

// RNE_f32(S / nb) for S = sum_j csum[j] * 2^(32j) in units of 2^-149 (csum[j] < 2^63).
QL_DEV float mean_from_limbs(const unsigned long long *csum, int64_t nb) {
  uint32_t S[kLimbs];
  unsigned long long carry = 0;
  for (int j = 0; j < kLimbs; ++j) {
    const unsigned long long t = csum[j] + carry;
    S[j] = (uint32_t)t;
    carry = t >> 32;
  }
  int top = kLimbs - 1;
  while (top >= 0 && S[top] == 0) --top;
  if (top < 0) return 0.0f;
  const int bitsS = 32 * top + 32 - __builtin_clz(S[top]);
  // W = S >> e keeps the top 96 bits; sticky0 records whether anything below was dropped
  const int e = bitsS > 96 ? bitsS - 96 : 0;
  const int q = e >> 5, r = e & 31;
  uint32_t W[3];
  for (int k = 0; k < 3; ++k) {
    const uint32_t lo = (k + q < kLimbs) ? S[k + q] : 0u;
    const uint32_t hi = (k + q + 1 < kLimbs) ? S[k + q + 1] : 0u;
    W[k] = r ? ((lo >> r) | (hi << (32 - r))) : lo;
  }
  bool sticky0 = r ? (S[q] & ((1u << r) - 1u)) != 0u : false;
  for (int k = 0; k < q; ++k) sticky0 = sticky0 || S[k] != 0u;
  // Q = W / nb, rem = W % nb (96-bit by 32-bit long division)
  const uint32_t den = (uint32_t)nb;
  uint32_t Q[3];
  unsigned long long rem = 0;
  for (int k = 2; k >= 0; --k) {
    const unsigned long long cur = (rem << 32) | W[k];
    Q[k] = (uint32_t)(cur / den);
    rem = cur % den;
  }
  const unsigned __int128 Qv = ((unsigned __int128)Q[2] << 64) | ((unsigned __int128)Q[1] << 32) | Q[0];
  int bitsQ = 0;
  for (int k = 2; k >= 0; --k)
    if (Q[k]) { bitsQ = 32 * k + 32 - __builtin_clz(Q[k]); break; }
  if (bitsQ == 0) {  // S/nb < 2^-149 * 1: rounds to 0 or the smallest denormal
    const bool up = 2 * rem > den || (2 * rem == den && sticky0);
    return up ? ldexpf(1.0f, -149) : 0.0f;
  }
  // value = (Q + frac) * 2^(e - 149); leading bit exponent E, float32 quantum 2^qe
  const int E = bitsQ - 1 + e - 149;
  const int qe = E - 23 > -149 ? E - 23 : -149;
  const int drop = qe - (e - 149);  // >= 0: bits of Q below the quantum
  unsigned long long mant = (unsigned long long)(Qv >> drop);
  bool up;
  if (drop == 0) {  // only when e == 0, so nothing below the remainder
    up = 2 * rem > den || (2 * rem == den && (mant & 1ull));
  } else {
    const bool half = (Qv >> (drop - 1)) & 1;
    const bool lower = (drop > 1 && (Qv & (((unsigned __int128)1 << (drop - 1)) - 1)) != 0) || rem != 0 || sticky0;
    up = half && (lower || (mant & 1ull));
  }
  if (up) ++mant;
  return ldexpf((float)mant, qe);
}

// Exact sum of this workgroup's share of the scales -> partial[blockIdx.x][kLimbs].
__global__ __launch_bounds__(256) void dq_partial_kernel(const float *__restrict__ absmax, int64_t nb,
                                                         unsigned long long *__restrict__ partial) {
  __shared__ unsigned long long bins[kNumBins];
  __shared__ unsigned long long limbs[kLimbs];
  for (int i = threadIdx.x; i < kNumBins; i += blockDim.x) bins[i] = 0ull;
  if (threadIdx.x < kLimbs) limbs[threadIdx.x] = 0ull;
  __syncthreads();

  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  int anchor = -1;
  unsigned long long acc = 0ull;
  // Branch-free except for the (rare) out-of-window atomic.  A zero has m == 0:
  // it adds nothing wherever it lands and never anchors the window.
  auto add = [&](float a) {
    uint32_t m;
    int sh;
    split_f32(a, m, sh);
    anchor = (anchor < 0 && m != 0u) ? (sh > 3 ? sh - 3 : 0) : anchor;
    const uint32_t d = (uint32_t)(sh - anchor);
    const bool in = d < 8u;
    acc += in ? (unsigned long long)(m << (d & 7u)) : 0ull;
    if (!in && m != 0u) atomicAdd(&bins[sh], (unsigned long long)m);
  };
  // 16-byte loads, four in flight per thread
  const int64_t nvec = nb >> 2;
  const f32x4 *v4 = reinterpret_cast<const f32x4 *>(absmax);
  for (int64_t i = tid; i < nvec; i += 4 * nthr) {
    f32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = (i + u * nthr < nvec) ? v4[i + u * nthr] : f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) add(x[u][k]);  // zero padding adds nothing
  }
  for (int64_t i = (nvec << 2) + tid; i < nb; i += nthr) add(absmax[i]);
  if (anchor >= 0 && acc) atomicAdd(&bins[anchor], acc);
  __syncthreads();
  // bin s holds v * 2^s (units of 2^-149), i.e. bits [s, s + 64): pieces of limbs s/32 .. s/32 + 2
  for (int s = threadIdx.x; s < kNumBins; s += blockDim.x) {
    const unsigned long long v = bins[s];
    if (!v) continue;
    const int a = s >> 5, b = s & 31;
    const unsigned long long lo = v << b;                       // low 64 bits of v * 2^b
    const unsigned long long hi = b ? (v >> (64 - b)) : 0ull;  // the bits above them
    atomicAdd(&limbs[a], lo & 0xFFFFFFFFull);
    atomicAdd(&limbs[a + 1], lo >> 32);
    if (hi) atomicAdd(&limbs[a + 2], hi);
  }
  __syncthreads();
  if (threadIdx.x < kLimbs) partial[(int64_t)blockIdx.x * kLimbs + threadIdx.x] = limbs[threadIdx.x];
}

// One wave per chunk of 256 scales: c = fp32(a - mean); s2 = fp32(max|c| / 127);
// q = rint(fp32(c / s2)) clamped to [-127, 127]; s2 == 0 gives q = 0.
__global__ __launch_bounds__(256) void dq_chunks_kernel(const float *__restrict__ absmax, int64_t nb,
                                                        const unsigned long long *__restrict__ partial,
                                                        int nparts, int8_t *__restrict__ qabsmax,
                                                        float *__restrict__ scale2, float *__restrict__ mean_out) {
  __shared__ unsigned long long csum[kLimbs];
  __shared__ float mean_s;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t nch = (nb + kChunk - 1) / kChunk;
  const int64_t cstep = (int64_t)gridDim.x * 4;
  int64_t chunk = (int64_t)blockIdx.x * 4 + (tid >> 6);
  // this lane's four scales of its first chunk, in flight while the mean is formed
  auto load4 = [&](int64_t ch, float (&a)[4]) {
    const int64_t i0 = ch * kChunk + lane * 4;
    if (ch < nch && i0 + 4 <= nb) {
      const f32x4 v = *reinterpret_cast<const f32x4 *>(absmax + i0);
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = v[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) a[k] = (ch < nch && i0 + k < nb) ? absmax[i0 + k] : 0.0f;
    }
  };
  float a[4];
  load4(chunk, a);
  if (tid < kLimbs) csum[tid] = 0ull;
  __syncthreads();
  constexpr int kLanesPerLimb = 256 / kLimbs;  // 21
  if (tid < kLanesPerLimb * kLimbs) {
    // the slots were written by other workgroups (other L2s): eight loads in flight
    // per step rather than one dependent load per slot
    const int j = tid % kLimbs;
    unsigned long long t = 0;
    for (int p = tid / kLimbs; p < nparts; p += 8 * kLanesPerLimb) {
      unsigned long long v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pu = p + u * kLanesPerLimb;
        v[u] = pu < nparts ? partial[(int64_t)pu * kLimbs + j] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) t += v[u];
    }
    if (t) atomicAdd(&csum[j], t);
  }
  __syncthreads();
  if (tid == 0) {
    mean_s = mean_from_limbs(csum, nb);
    if (blockIdx.x == 0) *mean_out = mean_s;
  }
  __syncthreads();
  const float mu = mean_s;
  for (; chunk < nch; chunk += cstep) {
    const int64_t i0 = chunk * kChunk + lane * 4;
    float c[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = (i0 + k < nb) ? a[k] - mu : 0.0f;
    float m = fmaxf(fmaxf(fabsf(c[0]), fabsf(c[1])), fmaxf(fabsf(c[2]), fabsf(c[3])));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    const float s2 = m / 127.0f;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      int q = 0;
      if (s2 != 0.0f) {
        float r = rintf(c[k] / s2);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        q = (int)r;
      }
      word |= ((uint32_t)(q & 0xFF)) << (8 * k);
    }
    if (i0 + 4 <= nb) {
      *reinterpret_cast<uint32_t *>(qabsmax + i0) = word;
    } else {
      for (int k = 0; k < 4; ++k)
        if (i0 + k < nb) qabsmax[i0 + k] = (int8_t)(word >> (8 * k));
    }
    if (lane == 0) scale2[chunk] = s2;
    if (chunk + cstep < nch) load4(chunk + cstep, a);
  }
}

// ---------------------------------------------------------------------------
// Dequantization ([MC] "1. NormalFloat": dequantize to BF16 before the
// matmul; [GO] "The core move").  A unit is one 32-bit word of codes = 8
// weights (inside one 64-block, so one a_hat).  Consecutive lanes take
// consecutive units, so each wave's code loads read 256 contiguous bytes and
// its 16-byte bf16 stores (or pairs of 16-byte float32 stores) write
// contiguous memory.  Each thread handles kDeqUnroll units per pass with all
// loads issued first.  A 256-entry LDS table at offset 0 maps a code byte to
// (level[high nibble], level[low nibble]): one shifted byte is the address and
// one 8-byte read returns both levels.
// ---------------------------------------------------------------------------

constexpr int kDeqUnroll = 8;

template <bool kOutBf16>
QL_DEV void dequant_unit(const f32x2 *lut, uint32_t cw, float ah, int64_t e0, int64_t n, void *__restrict__ out) {
  float wv[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const f32x2 l = lut[(cw >> (8 * b)) & 0xFF];
    wv[2 * b] = l[0] * ah;
    wv[2 * b + 1] = l[1] * ah;
  }
  if (e0 + 8 <= n) {
    if (kOutBf16) {
      // written once and not read again by this kernel: non-temporal stores
      __builtin_nontemporal_store(u32x4{pack_bf16x2(wv[0], wv[1]), pack_bf16x2(wv[2], wv[3]),
                                        pack_bf16x2(wv[4], wv[5]), pack_bf16x2(wv[6], wv[7])},
                                  reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + e0));
    } else {
      f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + e0);
      __builtin_nontemporal_store(f32x4{wv[0], wv[1], wv[2], wv[3]}, o);
      __builtin_nontemporal_store(f32x4{wv[4], wv[5], wv[6], wv[7]}, o + 1);
    }
  } else {
    for (int i = 0; i < 8; ++i) {
      if (e0 + i >= n) break;
      if (kOutBf16) reinterpret_cast<uint16_t *>(out)[e0 + i] = (uint16_t)(pack_bf16x2(wv[i], 0.0f) & 0xFFFF);
      else reinterpret_cast<float *>(out)[e0 + i] = wv[i];
    }
  }
}

template <bool kOutBf16, bool kNoDq>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ codes,
                                                         const int8_t *__restrict__ qabsmax,
                                                         const float *__restrict__ scale2,
                                                         const float *__restrict__ mean_in, int64_t n,
                                                         void *__restrict__ out, Nf4Tables tab,
                                                         const float *__restrict__ absmax) {
  // kNoDq: no double quantization, the float32 block scales (absmax) are used as stored
  __shared__ f32x2 lut[256];
  lut[threadIdx.x] = f32x2{tab.level[threadIdx.x >> 4], tab.level[threadIdx.x & 15]};
  __syncthreads();
  constexpr bool nodq = kNoDq;
  const float mu = nodq ? 0.0f : *mean_in;
  const int64_t nunits = (n + 7) / 8;
  const int64_t nbytes = (n + 1) / 2;
  const int64_t per_block = (int64_t)kDeqUnroll * blockDim.x;
  for (int64_t base = (int64_t)blockIdx.x * per_block; base < nunits; base += (int64_t)gridDim.x * per_block) {
    uint32_t cw[kDeqUnroll];
    int8_t q[kDeqUnroll];
    float s2[kDeqUnroll];
#pragma unroll
    for (int u = 0; u < kDeqUnroll; ++u) {
      const int64_t unit = base + u * blockDim.x + threadIdx.x;
      const int64_t e0 = unit * 8;
      cw[u] = 0x77777777u;
      q[u] = 0;
      s2[u] = 0.0f;
      if (unit < nunits) {
        const int64_t blk = e0 >> 6;
        if constexpr (nodq) {
          s2[u] = absmax[blk];  // used as a_hat directly below
        } else {
          q[u] = qabsmax[blk];
          s2[u] = scale2[blk / kChunk];
        }
        if (e0 + 8 <= n) {
          cw[u] = *reinterpret_cast<const uint32_t *>(codes + (e0 >> 1));
        } else {
          uint32_t t = 0x77777777u;
          for (int bb = 0; bb < 4; ++bb)
            if ((e0 >> 1) + bb < nbytes)
              t = (t & ~(0xFFu << (8 * bb))) | ((uint32_t)codes[(e0 >> 1) + bb] << (8 * bb));
          cw[u] = t;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDeqUnroll; ++u) {
      const int64_t unit = base + u * blockDim.x + threadIdx.x;
      if (unit < nunits)
        dequant_unit<kOutBf16>(lut, cw[u], nodq ? s2[u] : scale_hat(q[u], s2[u], mu), unit * 8, n, out);
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

static int grid_for(int64_t work_items, int per_block, int max_blocks) {
  int64_t g = (work_items + per_block - 1) / per_block;
  if (g < 1) g = 1;
  if (g > max_blocks) g = max_blocks;
  return (int)g;
}

hipError_t launch_quantize(const void *w, bool bf16, int64_t n, uint8_t *codes, float *absmax,
                           const Nf4Tables &tab, hipStream_t st) {
  // 512 weights per wave-iteration, 4 waves per block
  const int grid = grid_for((n + 511) / 512, 4, 256 * 32);
  return bf16 ? launch(quantize_kernel<true>, grid, 256, st, w, n, codes, absmax, tab)
              : launch(quantize_kernel<false>, grid, 256, st, w, n, codes, absmax, tab);
}

size_t dq_workspace_bytes() { return ((size_t)kDqGrid * kLimbs * 8 + 255) / 256 * 256; }

// The partial-sum slots of the allocation-free double quantization: one slot of
// kLimbs limbs per partial-sum workgroup, whatever the number of scales (the
// partial pass never has more than kDqGrid workgroups).  48 KB on every GPU the
// library runs on, held until the process ends.  Every slot a call's chunk pass
// reads is written by the same call's partial pass first, so nothing is cleared;
// calls that overlap on one GPU race on it.
static __device__ __align__(256) unsigned long long scratch[kDqGrid * kLimbs];

namespace {
std::mutex g_scratch_mu;
std::vector<unsigned long long *> g_scratch_ptr;  // per device: the device address of `scratch`
}  // namespace

hipError_t dq_scratch(hipStream_t st, unsigned long long **out) {
  int cur = -1, sdev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  e = hipStreamGetDevice(st, &sdev);
  if (e != hipSuccess) return e;
  if (sdev != cur) return hipErrorInvalidDevice;  // the kernels must see this device's copy
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= cur) g_scratch_ptr.resize(cur + 1, nullptr);
  if (!g_scratch_ptr[cur]) {
    // in host code `scratch` names a host-side stand-in: the device copy's address
    // comes from the runtime, once per device, with that device current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[cur] = reinterpret_cast<unsigned long long *>(p);
  }
  *out = g_scratch_ptr[cur];
  return hipSuccess;
}

hipError_t launch_double_quant_noalloc(const float *absmax, int64_t nb, int8_t *qabsmax, float *scale2,
                                       float *mean, hipStream_t st) {
  unsigned long long *ws = nullptr;
  const hipError_t e = dq_scratch(st, &ws);
  if (e != hipSuccess) return e;
  return launch_double_quant(absmax, nb, qabsmax, scale2, mean, ws, st);
}

hipError_t launch_double_quant(const float *absmax, int64_t nb, int8_t *qabsmax, float *scale2,
                               float *mean, void *ws, hipStream_t st) {
  auto *partial = reinterpret_cast<unsigned long long *>(ws);
  const int grid = grid_for(nb, 256 * 16, kDqGrid);
  const hipError_t e = launch(dq_partial_kernel, grid, 256, st, absmax, nb, partial);
  if (e != hipSuccess) return e;
  const int64_t nch = (nb + kChunk - 1) / kChunk;
  const int cgrid = grid_for(nch, 4, kDqChGrid);
  return launch(dq_chunks_kernel, cgrid, 256, st, absmax, nb, (const unsigned long long *)partial, grid, qabsmax,
                scale2, mean);
}

template <int MODE>
static hipError_t launch_merge_rq(int rq, dim3 grid, const MergeParams &p, const Nf4Tables &tab, hipStream_t st) {
  switch (rq) {
    case 0: return launch(merge_kernel<MODE, 0>, grid, 256, st, p, tab);
    case 1: return launch(merge_kernel<MODE, 1>, grid, 256, st, p, tab);
    case 2: return launch(merge_kernel<MODE, 2>, grid, 256, st, p, tab);
    case 3: return launch(merge_kernel<MODE, 3>, grid, 256, st, p, tab);
    default: return launch(merge_kernel<MODE, 4>, grid, 256, st, p, tab);
  }
}

hipError_t launch_merge(const MergeArgs &m, int mode, const Nf4Tables &tab, hipStream_t st) {
  MergeParams p{};
  p.codes = m.codes; p.qabsmax = m.qabsmax; p.scale2 = m.scale2; p.mean = m.mean;
  p.h = m.h; p.o = m.o; p.L1 = m.L1; p.L2 = m.L2; p.r = m.r; p.s = m.s;
  p.out = m.out; p.codes_out = m.codes_out; p.absmax_out = m.absmax_out;
  // about 2048 workgroups: strips of 64 rows x a range of k tiles
  const int64_t strips = m.o / 64, ktiles = m.h / 64;
  int64_t ksplit = (2048 + strips - 1) / strips;
  ksplit = ksplit < 1 ? 1 : (ksplit > ktiles ? ktiles : ksplit);
  p.kper = (int)((ktiles + ksplit - 1) / ksplit);
  ksplit = (ktiles + p.kper - 1) / p.kper;
  const dim3 grid((unsigned)strips, (unsigned)ksplit);
  const int rq = (m.r + 31) / 32;
  if (mode == 0) return launch_merge_rq<0>(rq, grid, p, tab, st);
  if (mode == 1) return launch_merge_rq<1>(rq, grid, p, tab, st);
  return launch_merge_rq<2>(rq, grid, p, tab, st);
}

hipError_t launch_dequantize(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                             const float *mean, int64_t n, void *out, bool bf16, const Nf4Tables &tab,
                             hipStream_t st, const float *absmax) {
  const int grid = grid_for((n + 7) / 8, 256 * kDeqUnroll, 256 * 16);
  auto k = absmax ? (bf16 ? dequantize_kernel<true, true> : dequantize_kernel<false, true>)
                  : (bf16 ? dequantize_kernel<true, false> : dequantize_kernel<false, false>);
  return launch(k, grid, 256, st, codes, qabsmax, scale2, mean, n, out, tab, absmax);
}

}  // namespace ql

// NF4 codec kernels for gfx950: blockwise quantization, double quantization
// of the block scales, dequantization.  All bandwidth-bound: every kernel
// streams its inputs once with 16-byte loads and writes its outputs once with
// coalesced stores.  Compiled with -ffp-contract=off so that every float32
// operation written below rounds separately, as the method's steps state.

#include "codec.h"

namespace ql {

// ---------------------------------------------------------------------------
// Blockwise NF4 quantization ([MC] "1. NormalFloat"; [TT] §2 "Choose a scale,
// then round", §3; blocks of 64: [MC] "2. Double quantization").
//
// Lane layout: each lane owns 8 consecutive weights, so the 8 lanes of a
// half-row own one 64-weight block.  The block's largest magnitude is reduced
// with three DPP max steps inside the 8-lane group.  Each weight's code comes
// from the bucket table (see nf4_tables.cpp): y = fma(w, 16/absmax, 16),
// bucket floor(y), one comparison against the bucket's guard band.  A lane
// with any weight inside a guard band, or a block whose scale is 0 or outside
// [2^-100, 2^100], recomputes its 8 codes with the IEEE division.  The 8 codes
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

template <bool kBf16>
QL_DEV void load8(const void *w, int64_t e0, int64_t n, float v[8]) {
  if (e0 + 8 <= n) {
    if (kBf16) {
      u32x4 d = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(w) + e0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_lo(d[i]);
        v[2 * i + 1] = bf16_hi(d[i]);
      }
    } else {
      const f32x4 *p = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(w) + e0);
      f32x4 a = p[0], b = p[1];
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

  for (int64_t base = wave * 512; base < n; base += nwaves * 512) {
    const int64_t e0 = base + lane * 8;
    float v[8];
    load8<kBf16>(w, e0, n, v);
    float m = fmaxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))),
                    fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7]))));
    const float a = dpp_max8(m);

    bool slow = !(a >= 0x1p-100f && a <= 0x1p100f);
    const float r16 = 16.0f * __builtin_amdgcn_rcpf(a);
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y = __builtin_fmaf(v[i], r16, 16.0f);
      uint32_t idx = (uint32_t)(int32_t)y;
      idx = idx > 32u ? 32u : idx;
      const EncBucket e = lut[idx];
      const bool up = y > e.hi;
      slow |= (y > e.lo) && !up;
      uint32_t c = e.base + (up ? 1u : 0u);
      // element i goes to byte i/2; even i in the high nibble
      word |= c << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
    }
    if (slow) {
      word = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float x = a > 0.0f ? v[i] / a : 0.0f;
        word |= exact_code(x, tab) << (8 * (i >> 1) + ((i & 1) ? 0 : 4));
      }
    }
    const int64_t c0 = e0 >> 1;  // first byte index of this lane
    if (e0 + 8 <= n) {
      *reinterpret_cast<uint32_t *>(codes + c0) = word;
    } else if (e0 < n) {
      // tail: pad codes beyond n are code 7 (zero level), bytes beyond ceil(n/2) untouched
      for (int i = 0; i < 8; ++i)
        if (e0 + i >= n) word = (word & ~(0xFu << (8 * (i >> 1) + ((i & 1) ? 0 : 4)))) |
                                (7u << (8 * (i >> 1) + ((i & 1) ? 0 : 4)));
      for (int b = 0; b < 4; ++b)
        if (c0 + b < ncodes) codes[c0 + b] = (uint8_t)(word >> (8 * b));
    }
    if ((lane & 7) == 0 && e0 < n) absmax[e0 >> 6] = a;
  }
}

// ---------------------------------------------------------------------------
// Double quantization ([MC] "2. Double quantization"; [TT] §6 and §2's
// symmetric int8 scheme).
//
// The mean of the block scales is computed exactly: every float32 is an
// integer multiple of 2^-149, so the sum is an integer that the kernels
// accumulate without rounding, binned by exponent, and the one rounding
// happens at the very end (dq_mean_finish).  Each lane keeps a private 64-bit
// accumulator for an 8-exponent window anchored at its first value; a value
// outside the window goes straight to its exponent bin.  Bins live in LDS per
// workgroup and are flushed to a global array of uint64 bins with atomics.
// Integer addition is associative, so the result does not depend on the order.
// ---------------------------------------------------------------------------

constexpr int kNumBins = 264;  // bin s holds integers in units of 2^(s-149)

__global__ void zero_u64_kernel(unsigned long long *p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

QL_DEV void split_f32(float a, uint32_t &mant, int &shift) {
  uint32_t b = __builtin_bit_cast(uint32_t, a);
  uint32_t e = (b >> 23) & 0xFF;
  mant = (b & 0x7FFFFFu) | (e ? 0x800000u : 0u);
  shift = e ? (int)e - 1 : 0;  // value = mant * 2^(shift - 149)
}

__global__ __launch_bounds__(256) void dq_bins_kernel(const float *__restrict__ absmax, int64_t nb,
                                                      unsigned long long *__restrict__ gbins) {
  __shared__ unsigned long long bins[kNumBins];
  for (int i = threadIdx.x; i < kNumBins; i += blockDim.x) bins[i] = 0ull;
  __syncthreads();

  const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t nthr = (int64_t)gridDim.x * blockDim.x;
  int anchor = -1;
  unsigned long long acc = 0ull;
  for (int64_t i = tid; i < nb; i += nthr) {
    uint32_t m;
    int s;
    split_f32(absmax[i], m, s);
    if (anchor < 0) anchor = s > 3 ? s - 3 : 0;
    const int d = s - anchor;
    if (d >= 0 && d < 8) {
      acc += (unsigned long long)(m << d);
    } else {
      atomicAdd(&bins[s], (unsigned long long)m);
    }
  }
  if (anchor >= 0 && acc) atomicAdd(&bins[anchor], acc);
  __syncthreads();
  for (int i = threadIdx.x; i < kNumBins; i += blockDim.x)
    if (bins[i]) atomicAdd(&gbins[i], bins[i]);
}

// One thread: mean = RNE_f32( (sum_s bins[s] * 2^(s-149)) / nb ).
__global__ void dq_mean_finish_kernel(const unsigned long long *__restrict__ gbins, int64_t nb,
                                      float *__restrict__ mean_out) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  // S in units of 2^-149 as little-endian 32-bit limbs; S < 2^32 * 2^31 * 2^263 < 2^326.
  constexpr int NL = 14;
  uint32_t S[NL];
  for (int i = 0; i < NL; ++i) S[i] = 0;
  for (int s = 0; s < kNumBins; ++s) {
    unsigned long long v = gbins[s];
    if (!v) continue;
    int limb = s >> 5, sh = s & 31;
    // add v << sh (up to 96 bits) at limb
    unsigned long long lo = (v << sh) & 0xFFFFFFFFull;
    unsigned long long mid = (sh ? (v >> (32 - sh)) : (v >> 32)) & 0xFFFFFFFFull;
    unsigned long long hi = sh ? (v >> (64 - sh)) : 0ull;
    unsigned long long carry = 0;
    unsigned long long parts[3] = {lo, mid, hi};
    for (int k = 0; limb + k < NL; ++k) {
      unsigned long long add = (k < 3 ? parts[k] : 0ull) + carry;
      if (k >= 3 && add == 0) break;
      unsigned long long t = (unsigned long long)S[limb + k] + add;
      S[limb + k] = (uint32_t)t;
      carry = t >> 32;
    }
  }
  int top = NL - 1;
  while (top >= 0 && S[top] == 0) --top;
  if (top < 0) { *mean_out = 0.0f; return; }
  const int bitsS = top * 32 + (32 - __builtin_clz(S[top]));
  const uint32_t den = (uint32_t)nb;
  const int bitsD = 32 - __builtin_clz(den);
  // scale S by 2^k so the quotient has at least 27 bits
  int k = 27 + bitsD - bitsS;
  if (k < 0) k = 0;
  uint32_t X[NL + 3];
  for (int i = 0; i < NL + 3; ++i) X[i] = 0;
  {
    const int limb = k >> 5, sh = k & 31;
    for (int i = 0; i < NL; ++i) {
      unsigned long long v = (unsigned long long)S[i] << sh;
      if (i + limb < NL + 3) X[i + limb] |= (uint32_t)v;
      if (i + limb + 1 < NL + 3) X[i + limb + 1] |= (uint32_t)(v >> 32);
    }
  }
  // long division X / den
  uint32_t Q[NL + 3];
  unsigned long long rem = 0;
  for (int i = NL + 2; i >= 0; --i) {
    unsigned long long cur = (rem << 32) | X[i];
    Q[i] = (uint32_t)(cur / den);
    rem = cur % den;
  }
  int qt = NL + 2;
  while (qt > 0 && Q[qt] == 0) --qt;
  const int bitsQ = qt * 32 + (32 - __builtin_clz(Q[qt]));
  // value = Q * 2^(-k-149) (+ fraction rem/den); exponent E with 2^E <= value
  const int E = bitsQ - 1 - k - 149;
  int qe = E - 23;
  if (qe < -149) qe = -149;
  const int drop = qe + k + 149;  // bits of Q below the float32 quantum (>= 3 by choice of k)
  auto bit = [&](int p) -> uint32_t { return (p < 0) ? 0u : ((Q[p >> 5] >> (p & 31)) & 1u); };
  unsigned long long mant = 0;
  for (int p = bitsQ - 1; p >= drop; --p) mant = (mant << 1) | bit(p);
  const uint32_t half = bit(drop - 1);
  bool sticky = rem != 0;
  for (int p = drop - 2; p >= 0 && !sticky; --p) sticky = bit(p) != 0;
  if (half && (sticky || (mant & 1ull))) ++mant;
  *mean_out = ldexpf((float)mant, qe);
}

// One wave per chunk of 256 scales: c = fp32(a - mean); s2 = fp32(max|c| / 127);
// q = rint(fp32(c / s2)) clamped to [-127, 127]; s2 == 0 gives q = 0.
__global__ __launch_bounds__(256) void dq_chunks_kernel(const float *__restrict__ absmax, int64_t nb,
                                                        const float *__restrict__ mean_in,
                                                        int8_t *__restrict__ qabsmax,
                                                        float *__restrict__ scale2) {
  const int lane = threadIdx.x & 63;
  const int64_t chunk = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int64_t nch = (nb + kChunk - 1) / kChunk;
  if (chunk >= nch) return;
  const float mu = *mean_in;
  const int64_t i0 = chunk * kChunk + lane * 4;
  float c[4];
  if (i0 + 4 <= nb) {
    f32x4 a = *reinterpret_cast<const f32x4 *>(absmax + i0);
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = a[k] - mu;
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = (i0 + k < nb) ? absmax[i0 + k] - mu : 0.0f;
  }
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
}

// ---------------------------------------------------------------------------
// Dequantization ([MC] "1. NormalFloat": dequantize to BF16 before the
// matmul; [GO] "The core move").  Each lane turns 16 bytes of codes (32
// weights, all in one 64-block) into 32 float32 or bf16 values.  The 16
// levels sit in LDS at a 16-byte stride, so the high nibble of a byte,
// masked in place, is already its table offset; different codes hit
// different banks and equal codes broadcast.
// ---------------------------------------------------------------------------

template <bool kOutBf16>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint8_t *__restrict__ codes,
                                                         const int8_t *__restrict__ qabsmax,
                                                         const float *__restrict__ scale2,
                                                         const float *__restrict__ mean_in, int64_t n,
                                                         void *__restrict__ out, Nf4Tables tab) {
  __shared__ float lut[16 * 4];
  if (threadIdx.x < 64) lut[threadIdx.x] = tab.level[threadIdx.x >> 2];
  __syncthreads();
  const float mu = *mean_in;
  const int64_t ngroups = (n + 31) / 32;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < ngroups; g += stride) {
    const int64_t e0 = g * 32;
    const int64_t blk = e0 >> 6;
    const float ah = scale_hat(qabsmax[blk], scale2[blk / kChunk], mu);
    u32x4 cw;
    if (e0 + 32 <= n) {
      cw = *reinterpret_cast<const u32x4 *>(codes + (e0 >> 1));
    } else {
      const int64_t nbytes = (n + 1) / 2;
      uint32_t t[4] = {0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
      for (int b = 0; b < 16; ++b)
        if ((e0 >> 1) + b < nbytes)
          t[b >> 2] = (t[b >> 2] & ~(0xFFu << (8 * (b & 3)))) | ((uint32_t)codes[(e0 >> 1) + b] << (8 * (b & 3)));
      cw = u32x4{t[0], t[1], t[2], t[3]};
    }
    float wv[32];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t hi = cw[d] & 0xF0F0F0F0u;        // high nibbles * 16
      const uint32_t lo = (cw[d] << 4) & 0xF0F0F0F0u; // low nibbles * 16
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const float l_hi = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + ((hi >> (8 * b)) & 0xFF));
        const float l_lo = *reinterpret_cast<const float *>(reinterpret_cast<const char *>(lut) + ((lo >> (8 * b)) & 0xFF));
        wv[8 * d + 2 * b] = l_hi * ah;
        wv[8 * d + 2 * b + 1] = l_lo * ah;
      }
    }
    if (e0 + 32 <= n) {
      if (kOutBf16) {
        u32x4 *o = reinterpret_cast<u32x4 *>(reinterpret_cast<uint16_t *>(out) + e0);
#pragma unroll
        for (int q = 0; q < 4; ++q)
          o[q] = u32x4{pack_bf16x2(wv[8 * q], wv[8 * q + 1]), pack_bf16x2(wv[8 * q + 2], wv[8 * q + 3]),
                       pack_bf16x2(wv[8 * q + 4], wv[8 * q + 5]), pack_bf16x2(wv[8 * q + 6], wv[8 * q + 7])};
      } else {
        f32x4 *o = reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(out) + e0);
#pragma unroll
        for (int q = 0; q < 8; ++q) o[q] = f32x4{wv[4 * q], wv[4 * q + 1], wv[4 * q + 2], wv[4 * q + 3]};
      }
    } else {
      for (int i = 0; i < 32; ++i) {
        if (e0 + i >= n) break;
        if (kOutBf16) {
          reinterpret_cast<uint16_t *>(out)[e0 + i] = (uint16_t)(pack_bf16x2(wv[i], 0.0f) & 0xFFFF);
        } else {
          reinterpret_cast<float *>(out)[e0 + i] = wv[i];
        }
      }
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
  if (bf16)
    quantize_kernel<true><<<grid, 256, 0, st>>>(w, n, codes, absmax, tab);
  else
    quantize_kernel<false><<<grid, 256, 0, st>>>(w, n, codes, absmax, tab);
  return hipGetLastError();
}

size_t dq_workspace_bytes() { return ((size_t)kNumBins * 8 + 255) / 256 * 256; }

hipError_t launch_double_quant(const float *absmax, int64_t nb, int8_t *qabsmax, float *scale2,
                               float *mean, void *ws, hipStream_t st) {
  auto *bins = reinterpret_cast<unsigned long long *>(ws);
  zero_u64_kernel<<<(kNumBins + 255) / 256, 256, 0, st>>>(bins, kNumBins);
  const int grid = grid_for(nb, 256 * 16, 1024);
  dq_bins_kernel<<<grid, 256, 0, st>>>(absmax, nb, bins);
  dq_mean_finish_kernel<<<1, 64, 0, st>>>(bins, nb, mean);
  const int64_t nch = (nb + kChunk - 1) / kChunk;
  dq_chunks_kernel<<<(int)((nch + 3) / 4), 256, 0, st>>>(absmax, nb, mean, qabsmax, scale2);
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                             const float *mean, int64_t n, void *out, bool bf16, const Nf4Tables &tab,
                             hipStream_t st) {
  const int grid = grid_for((n + 31) / 32, 256, 256 * 64);
  if (bf16)
    dequantize_kernel<true><<<grid, 256, 0, st>>>(codes, qabsmax, scale2, mean, n, out, tab);
  else
    dequantize_kernel<false><<<grid, 256, 0, st>>>(codes, qabsmax, scale2, mean, n, out, tab);
  return hipGetLastError();
}

}  // namespace ql

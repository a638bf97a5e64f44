// Shared device/host definitions for the gfx950 NF4 + LoRA kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#define QL_DEV __device__ __forceinline__

namespace ql {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;   // weights per first-level scale
constexpr int kChunk = 256;  // first-level scales per second-level step
constexpr int kWave = 64;

// Encoder bucket table: y = 16*x + yoff (yoff = 16 plus a shift in [0, 1)) for
// a normalised weight x in [-1, 1] falls in bucket floor(y) (0..33).  Each bucket holds at most one
// decision threshold; `lo`/`hi` bound its guard band (see nf4_tables.hip).
struct EncBucket {
  float hi;     // y > hi: code is base + 1 for certain
  float lo;     // y <= lo: code is base for certain
  float tx;     // the threshold in x units (largest float32 below the midpoint), for the exact path
  uint32_t base;
};

constexpr int kBuckets = 34;

// 4-bit codebooks: the index of a value in an ascending 16-entry table is its code.
constexpr int kCodebooks = 3;  // 0 NF4, 1 INT4 (symmetric absmax grid), 2 FP4 (E2M1 values)

struct Nf4Tables {
  float level[16];              // the codebook, ascending
  float thr[15];                // thr[j] = largest float32 <= midpoint(level[j], level[j+1])
  EncBucket bucket[kBuckets];
  float yoff;                   // y = 16 x + yoff
  uint32_t zero_code;           // the code of level 0 (padding)
};

// Built once per codebook on the host (nf4_tables.hip); passed to kernels by value.
const Nf4Tables *host_tables(int codebook = 0);  // nullptr if construction failed

// ---- small device helpers ------------------------------------------------

// Two float32 -> packed bf16 pair (round to nearest even), low half = a.
QL_DEV uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

QL_DEV float bf16_lo(uint32_t d) { return __builtin_bit_cast(float, d << 16); }
QL_DEV float bf16_hi(uint32_t d) { return __builtin_bit_cast(float, d & 0xFFFF0000u); }

// Scale reconstruction a_hat = fp32(fp32(q * s2) + mean), two roundings, no FMA.
// (The whole library is compiled with -ffp-contract=off.)
QL_DEV float scale_hat(int8_t q, float s2, float mean) {
  float p = (float)q * s2;
  return p + mean;
}

// ---- launches ------------------------------------------------------------

// Launch through hipLaunchKernel and return that launch's own status: a failed
// launch is reported without reading (or clearing) the calling thread's
// last-error state, which belongs to the caller.
template <typename... P, size_t... I>
hipError_t launch_tuple(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, std::tuple<P...> &t,
                        std::index_sequence<I...>) {
  void *args[] = {static_cast<void *>(&std::get<I>(t))...};
  return hipLaunchKernel(reinterpret_cast<const void *>(k), grid, block, args, 0, st);
}
template <typename... P, typename... A>
hipError_t launch(void (*k)(P...), dim3 grid, dim3 block, hipStream_t st, A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> t(a...);
  return launch_tuple(k, grid, block, st, t, std::index_sequence_for<P...>{});
}

}  // namespace ql

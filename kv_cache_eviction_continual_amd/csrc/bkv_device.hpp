// bkv_device.hpp -- device-side helpers shared by the libbkv kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv.h"

namespace bkv {

constexpr int kStatusWord = 0;        // int32 index of the device status word in ws
constexpr int kRowsMovedWord = 2;     // uint64 at byte offset 8 (int32 index 2)
constexpr size_t kHeaderBytes = 256;  // status + statistics block at the front of ws

// ---------------------------------------------------------------------------
// Storage element types
// ---------------------------------------------------------------------------

// Round a binary64 value once to bfloat16 (round to nearest, ties to even),
// working on the binary64 bit pattern: keep the top 8 significant bits of a
// normal bf16 result, or the bits above 2^-133 for a subnormal one.
__device__ inline uint16_t bf16_from_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t sign = (uint32_t)(u >> 63) << 15;
  const int ef = (int)((u >> 52) & 0x7FF);
  const uint64_t frac = u & ((1ull << 52) - 1);
  if (ef == 0x7FF) return frac ? (uint16_t)0x7FC0 : (uint16_t)(sign | 0x7F80);
  if (ef == 0) return (uint16_t)sign;  // |v| < 2^-1022: far below half the smallest bf16
  int e = ef - 1023;
  const uint64_t sig = frac | (1ull << 52);  // 53-bit significand, v = sig * 2^(e-52)
  if (e >= -126) {
    uint64_t keep = sig >> 45;  // 8 significant bits
    const uint64_t rem = sig & ((1ull << 45) - 1);
    const uint64_t half = 1ull << 44;
    if (rem > half || (rem == half && (keep & 1))) keep += 1;
    if (keep == 256) {
      keep = 128;
      e += 1;
    }
    if (e > 127) return (uint16_t)(sign | 0x7F80);
    return (uint16_t)(sign | ((uint32_t)(e + 127) << 7) | (uint32_t)(keep & 0x7F));
  }
  // subnormal result: count of 2^-133 units, sig * 2^(e-52+133) = sig >> (-81-e)
  const int sh = -81 - e;  // >= 46
  if (sh >= 54) return (uint16_t)sign;  // below a quarter unit: rounds to zero
  uint64_t keep = sig >> sh;
  const uint64_t rem = sig & ((1ull << sh) - 1);
  const uint64_t half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (keep & 1))) keep += 1;
  return (uint16_t)(sign | (uint32_t)keep);  // keep == 128 encodes 2^-126 exactly
}

template <int DT>
struct Elem;

template <>
struct Elem<BKV_F32> {
  using T = float;
  static constexpr int kBytes = 4;
  __device__ static inline float to_f32(T v) { return v; }
  __device__ static inline double to_f64(T v) { return (double)v; }
  __device__ static inline T from_f64(double v) { return (float)v; }  // RNE
};

template <>
struct Elem<BKV_BF16> {
  using T = uint16_t;
  static constexpr int kBytes = 2;
  __device__ static inline float to_f32(T v) { return __uint_as_float((uint32_t)v << 16); }
  __device__ static inline double to_f64(T v) { return (double)to_f32(v); }
  __device__ static inline T from_f64(double v) { return bf16_from_f64(v); }
};

// ---------------------------------------------------------------------------
// Small helpers
// ---------------------------------------------------------------------------

__device__ inline void set_status(int32_t* ws_words, int bit) {
  atomicOr(&ws_words[kStatusWord], bit);
}

// Strict order used by every argmin: smaller value, then smaller index.
__device__ inline bool better(double v, int i, double bv, int bi) {
  return v < bv || (v == bv && i < bi);
}

// Copy `nbytes` (a multiple of 16) from global memory to LDS with 16-byte
// accesses spread over the block.
__device__ inline void copy16(void* dst, const void* src, int nbytes, int tid, int nthreads) {
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(dst);
  for (int i = tid; i < nbytes / 16; i += nthreads) d[i] = s[i];
}

// Block-wide exclusive prefix sum of one int per thread; returns the prefix
// and writes the block total to *total.  `scratch` holds >= 16 ints of LDS.
__device__ inline int block_exclusive_scan(int v, int* scratch, int* total) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wave] = x;
  __syncthreads();
  int wave_base = 0, sum = 0;
  for (int w = 0; w < nwaves; ++w) {
    int t = scratch[w];
    if (w < wave) wave_base += t;
    sum += t;
  }
  __syncthreads();
  *total = sum;
  return wave_base + x - v;
}

}  // namespace bkv

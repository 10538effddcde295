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

// Round a binary64 value once to bfloat16 (round to nearest, ties to even).
// Every bfloat16 value, and every midpoint between two neighbours, is a
// binary32 number.  Rounding to binary32 first (to nearest) therefore never
// moves the value across such a midpoint: it either lands strictly inside the
// same half-interval, where the integer round-to-nearest-even of the binary32
// bits gives the right result, or exactly on a midpoint, where the binary64
// value decides the direction (ties to even only if it is the midpoint).
__device__ inline uint16_t bf16_from_f64(double v) {
  const float f = (float)v;
  if (f != f) return (uint16_t)0x7FC0;
  const uint32_t u = __float_as_uint(f);
  const uint32_t hi = u >> 16;
  if ((u & 0xFFFFu) == 0x8000u) {
    const double a = fabs(v), af = fabs((double)f);
    return (uint16_t)(a > af ? hi + 1 : (a < af ? hi : hi + (hi & 1)));
  }
  return (uint16_t)((u + 0x7FFFu + (hi & 1)) >> 16);
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

// decode.hip -- one decode step of attention for every (slot, KV head), with
// the probabilities of the step's queries optionally folded into a per-key
// running maximum (the recent-query capture).
//
// The eviction score takes the attention of the recent queries together with
// the beacons' (wzjinhao.cn news article 56682 on BeaconKV, section
// 信标查询怎么用); the same article (section 信标和最近查询该怎么分配) places
// the extra cost of scoring in the beacons' attention.  Decoding already
// computes each recent query's attention, so its probabilities can be kept as
// they are produced: capture[j] = max(capture[j], max_g p_g(j)), and at
// eviction only the beacons need a scoring pass.  A captured probability is
// normalised over the keys present at its own step.
//
// decode_kernel: one workgroup of four waves per (slot, KV head).  Sixteen
// lanes share a key (16-byte loads, one 64-byte row piece per lane group of
// a wave: four consecutive keys per wave and step), binary32 dot products
// reduced across the sixteen lanes, an online softmax per query head in the
// log2 domain, and the value rows accumulated under it.  The four key groups
// of a wave, then the four waves, are merged at the end.  With a capture
// array, each key's logits are kept (in LDS when the unit's G x Lmax of them
// fit in 48 KB, else in a workspace slice), and a last sweep turns them into
// probabilities with the final log-sum-exp and folds them in.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

constexpr int kDecThreads = 256;
constexpr int kDecSteps = 4;  // four-key steps per wave per block (64 keys per block)

struct DecU32x8 {
  uint4 a, b;
};

template <int BYTES>
struct DecRaw;
template <>
struct DecRaw<8> {
  using type = uint2;
};
template <>
struct DecRaw<16> {
  using type = uint4;
};
template <>
struct DecRaw<32> {
  using type = DecU32x8;
};

// Lane part p of a row holds elements [p EL, p EL + EL), EL = D / 16.
template <int DT, int D>
struct DecPart {
  using E = Elem<DT>;
  using T = typename E::T;
  static constexpr int EL = D / 16;
  using R = typename DecRaw<EL * (int)sizeof(T)>::type;
  struct Arr {
    T e[EL];
  };
  __device__ static inline R load(const T* row, int part) { return *reinterpret_cast<const R*>(row + part * EL); }
  __device__ static inline void widen(const R& r, float (&x)[EL]) {
    const Arr a = __builtin_bit_cast(Arr, r);
#pragma unroll
    for (int k = 0; k < EL; ++k) x[k] = E::to_f32(a.e[k]);
  }
};

// Sum over a row of sixteen lanes, left in every lane of the row, by DPP
// moves (no LDS): swap neighbours, swap pairs, mirror the halves of the row,
// mirror the row.  Each step adds two values in either order, so every lane
// ends with the same bits.
template <int CTRL>
__device__ inline float dec_dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ inline float dec_sum16(float v) {
  v += dec_dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dec_dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dec_dpp<0x141>(v);  // row_half_mirror
  v += dec_dpp<0x140>(v);  // row_mirror
  return v;
}

// exp2 of x - m for a running maximum m that may still be -inf (nothing seen).
__device__ inline float dec_rescale(float x, float m) { return m == -__builtin_huge_valf() ? 0.0f : exp2f(x - m); }

constexpr int kDecLdsLogits = 48 * 1024;  // bytes of logits kept in LDS at most

template <int DT, int D, int G, bool kLdsLogits>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(
    const typename Elem<DT>::T* __restrict__ q, const typename Elem<DT>::T* __restrict__ K,
    const typename Elem<DT>::T* __restrict__ V, const int32_t* __restrict__ len, int Hkv, int Lmax,
    float* __restrict__ out, float* __restrict__ capture, float* __restrict__ logits, int32_t* __restrict__ ws_words) {
  using P = DecPart<DT, D>;
  using T = typename Elem<DT>::T;
  constexpr int EL = P::EL;
  constexpr int NW = kDecThreads / 64;
  __shared__ float red_m[NW][G], red_l[NW][G];
  __shared__ float red_acc[NW][G][D];
  __shared__ float lse2[G];
  extern __shared__ float lds_logits[];  // [G][Lmax] when kLdsLogits

  const size_t unit = blockIdx.x;
  const int n = (int)(unit / Hkv);
  const int hkv = (int)(unit % Hkv);
  const int L = len[n];
  if (L < 0 || L > Lmax) {
    if (threadIdx.x == 0) set_status(ws_words, BKV_DEV_BAD_LEN);
    return;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = lane & 15, sub = lane >> 4;
  const float ninf = -__builtin_huge_valf();
  const float scale2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
  const T* Kb = K + unit * (size_t)Lmax * D;
  const T* Vb = V + unit * (size_t)Lmax * D;

  // this lane's part of every query of the group
  float qv[G][EL];
  const size_t qhead = (size_t)n * Hkv * G + (size_t)hkv * G;
#pragma unroll
  for (int g = 0; g < G; ++g) P::widen(P::load(q + (qhead + g) * D, part), qv[g]);

  float m[G], l[G], acc[G][EL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = ninf;
    l[g] = 0.0f;
#pragma unroll
    for (int k = 0; k < EL; ++k) acc[g][k] = 0.0f;
  }

  // the rows of the next block are loaded while this block is computed
  typename P::R kr[kDecSteps], vr[kDecSteps];
#pragma unroll
  for (int u = 0; u < kDecSteps; ++u) {
    const int j = 16 * u + 4 * wave + sub;
    if (j < L) {
      kr[u] = P::load(Kb + (size_t)j * D, part);
      vr[u] = P::load(Vb + (size_t)j * D, part);
    }
  }
  for (int j0 = 0; j0 < L; j0 += 16 * kDecSteps) {
    typename P::R kn[kDecSteps], vn[kDecSteps];
#pragma unroll
    for (int u = 0; u < kDecSteps; ++u) {
      const int j = j0 + 16 * kDecSteps + 16 * u + 4 * wave + sub;
      if (j < L) {
        kn[u] = P::load(Kb + (size_t)j * D, part);
        vn[u] = P::load(Vb + (size_t)j * D, part);
      }
    }
    float sv[kDecSteps][G];
#pragma unroll
    for (int u = 0; u < kDecSteps; ++u) {
      const int j = j0 + 16 * u + 4 * wave + sub;
      float x[EL];
      if (j < L) P::widen(kr[u], x);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float d = 0.0f;
        if (j < L) {
#pragma unroll
          for (int k = 0; k < EL; ++k) d = fmaf(x[k], qv[g][k], d);
        }
        d = dec_sum16(d);
        sv[u][g] = j < L ? d * scale2 : ninf;
        if (capture != nullptr && part == 0 && j < L) {
          if constexpr (kLdsLogits) lds_logits[g * Lmax + j] = sv[u][g];
          else logits[(unit * G + g) * (size_t)Lmax + j] = sv[u][g];
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float mb = sv[0][g];
#pragma unroll
      for (int u = 1; u < kDecSteps; ++u) mb = fmaxf(mb, sv[u][g]);
      const float m_new = fmaxf(m[g], mb);
      if (m_new == ninf) continue;  // no key of this lane group in the block yet
      const float corr = dec_rescale(m[g], m_new);
      l[g] *= corr;
#pragma unroll
      for (int k = 0; k < EL; ++k) acc[g][k] *= corr;
      m[g] = m_new;
    }
#pragma unroll
    for (int u = 0; u < kDecSteps; ++u) {
      const int j = j0 + 16 * u + 4 * wave + sub;
      if (j >= L) continue;
      float v[EL];
      P::widen(vr[u], v);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = __builtin_amdgcn_exp2f(sv[u][g] - m[g]);  // <= 1; a term below 2^-126 of it is 0
        l[g] += p;
#pragma unroll
        for (int k = 0; k < EL; ++k) acc[g][k] = fmaf(p, v[k], acc[g][k]);
      }
    }
#pragma unroll
    for (int u = 0; u < kDecSteps; ++u) {
      kr[u] = kn[u];
      vr[u] = vn[u];
    }
  }

  // merge the four key groups of the wave (lanes with the same part)
#pragma unroll
  for (int off = 16; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = __shfl_xor(m[g], off, 64);
      const float lo = __shfl_xor(l[g], off, 64);
      const float M = fmaxf(m[g], mo);
      const float ca = dec_rescale(m[g], M), cb = dec_rescale(mo, M);
      l[g] = l[g] * ca + lo * cb;
#pragma unroll
      for (int k = 0; k < EL; ++k) acc[g][k] = acc[g][k] * ca + __shfl_xor(acc[g][k], off, 64) * cb;
      m[g] = M;
    }
  }
  if (sub == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (part == 0) {
        red_m[wave][g] = m[g];
        red_l[wave][g] = l[g];
      }
#pragma unroll
      for (int k = 0; k < EL; ++k) red_acc[wave][g][part * EL + k] = acc[g][k];
    }
  }
  __syncthreads();
  // then the four waves: out = sum_w acc_w 2^(m_w - M) / sum_w l_w 2^(m_w - M)
  for (int t = threadIdx.x; t < G * D; t += kDecThreads) {
    const int g = t / D, dim = t - g * D;
    float M = ninf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][g]);
    float num = 0.0f, den = 0.0f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float c = dec_rescale(red_m[w][g], M);
      num = fmaf(red_acc[w][g][dim], c, num);
      den = fmaf(red_l[w][g], c, den);
    }
    out[(qhead + g) * D + dim] = den > 0.0f ? num / den : 0.0f;
    if (dim == 0) lse2[g] = den > 0.0f ? M + log2f(den) : __builtin_huge_valf();
  }
  if (capture == nullptr) return;  // uniform
  __syncthreads();  // lse2 and every key's logits are in place
  float* cap = capture + unit * (size_t)Lmax;
  for (int j = threadIdx.x; j < L; j += kDecThreads) {
    float c = cap[j];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s2 = kLdsLogits ? lds_logits[g * Lmax + j] : logits[(unit * G + g) * (size_t)Lmax + j];
      c = fmaxf(c, exp2f(s2 - lse2[g]));
    }
    cap[j] = c;
  }
}

template <int DT, int D, int G>
static hipError_t launch_decode_g(const void* q, const void* K, const void* V, const int32_t* len, int N, int Hkv,
                                  int Lmax, float* out, float* capture, float* logits, int32_t* ws_words,
                                  hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const size_t lds = (size_t)G * Lmax * sizeof(float);
  if (capture != nullptr && lds <= (size_t)kDecLdsLogits) {
    auto kern = decode_kernel<DT, D, G, true>;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(N * Hkv), dim3(kDecThreads), lds, st, (const ET*)q, (const ET*)K, (const ET*)V,
                       len, Hkv, Lmax, out, capture, logits, ws_words);
  } else {
    hipLaunchKernelGGL((decode_kernel<DT, D, G, false>), dim3(N * Hkv), dim3(kDecThreads), 0, st, (const ET*)q,
                       (const ET*)K, (const ET*)V, len, Hkv, Lmax, out, capture, logits, ws_words);
  }
  return hipGetLastError();
}

// G (query heads per KV head) in {1, 2, 4, 5, 8}.
template <int DT, int D>
hipError_t launch_decode(const void* q, const void* K, const void* V, const int32_t* len, int N, int Hkv, int G,
                         int Lmax, float* out, float* capture, float* logits, int32_t* ws_words, hipStream_t st) {
  switch (G) {
    case 1: return launch_decode_g<DT, D, 1>(q, K, V, len, N, Hkv, Lmax, out, capture, logits, ws_words, st);
    case 2: return launch_decode_g<DT, D, 2>(q, K, V, len, N, Hkv, Lmax, out, capture, logits, ws_words, st);
    case 4: return launch_decode_g<DT, D, 4>(q, K, V, len, N, Hkv, Lmax, out, capture, logits, ws_words, st);
    case 5: return launch_decode_g<DT, D, 5>(q, K, V, len, N, Hkv, Lmax, out, capture, logits, ws_words, st);
    case 8: return launch_decode_g<DT, D, 8>(q, K, V, len, N, Hkv, Lmax, out, capture, logits, ws_words, st);
    default: return hipErrorInvalidValue;
  }
}

#define BKV_INST_DECODE(DT, D)                                                                                 \
  template hipError_t launch_decode<DT, D>(const void*, const void*, const void*, const int32_t*, int, int, int, \
                                           int, float*, float*, float*, int32_t*, hipStream_t);
BKV_INST_DECODE(BKV_F32, 64)
BKV_INST_DECODE(BKV_F32, 128)
BKV_INST_DECODE(BKV_BF16, 64)
BKV_INST_DECODE(BKV_BF16, 128)

}  // namespace bkv

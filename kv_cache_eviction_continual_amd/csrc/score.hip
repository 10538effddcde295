// score.hip -- beacon-guided importance scores on gfx950 matrix cores.
//
// For one (slot, KV head) the observation rows are the recent queries and
// beacons of the G query heads of the group (already rotated and rounded by
// obs_build_kernel).  Each row r attends to every cached key:
//   p_r(j) = softmax_j(q_r . k_j / sqrt(d)),  score_j = max_r p_r(j)
// (inkeast.github.io MessageDaily paper-reading post on BeaconKV, sections 三
// and 4.4: scoring by the attention of recent queries together with the
// beacon set; wzjinhao.cn news article 56682, section 信标查询怎么用:
// aggregation by maximum).
//
// One workgroup per (slot, KV head), one wave per 32-row tile of
// observation rows, so the wave keeps its query fragment in registers for
// the whole kernel.  K streams through LDS in tiles of kTile keys (coalesced
// 16-byte loads, the next tile prefetched into registers while the current
// one is multiplied).  Two passes over K:
//   pass 1: S^T = K Q^T on MFMA (lane = row, 16 keys per lane), online
//           row max and sum of exp2 -> per-row log2-sum-exp;
//   pass 2: S = Q K^T on MFMA (lane = key, 16 rows per lane), per-key max of
//           (s - lse) over the wave's rows, then over the waves through LDS;
//           one exp2 per key.  Pass 2 walks the tiles in reverse so that the
//           most recently read tiles are still cached.
// exp(max_r(s_r - lse_r)) = max_r exp(s_r - lse_r), so one exp per key
// suffices.  Logits are accumulated in fp32 from exact bf16 (or fp32)
// products.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16_t;

constexpr int kTile = 128;   // keys per LDS tile
constexpr int kSub = 32;     // keys per MFMA sub-tile

// Per storage type: fragment of one MFMA k-step.
template <int DT, int D>
struct Mfma;

template <int D>
struct Mfma<BKV_BF16, D> {
  using Frag = bf16x8_t;
  static constexpr int kSteps = D / 16;
  // dims of lane `lane` at k-step s: 16 s + 8 (lane / 32) + [0, 8)
  __device__ static inline Frag load(const unsigned char* row, int s, int lane) {
    uint4 w = *reinterpret_cast<const uint4*>(row + (size_t)(16 * s + 8 * (lane >> 5)) * 2);
    return __builtin_bit_cast(Frag, w);
  }
  __device__ static inline floatx16_t mma(Frag a, Frag b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <int D>
struct Mfma<BKV_F32, D> {
  using Frag = float;
  static constexpr int kSteps = D / 2;
  // dim of lane `lane` at k-step s: 2 s + lane / 32
  __device__ static inline Frag load(const unsigned char* row, int s, int lane) {
    return *reinterpret_cast<const float*>(row + (size_t)(2 * s + (lane >> 5)) * 4);
  }
  __device__ static inline floatx16_t mma(Frag a, Frag b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Accumulator element r of lane l holds output row 8 (r / 4) + 4 (l / 32) +
// r % 4 and output column l % 32 (32x32 MFMA family, checked on gfx950).
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

template <int DT, int D>
struct ScoreLayout {
  static constexpr int kRowBytes = D * Elem<DT>::kBytes;
  static constexpr int kRowStride = kRowBytes + 16;
  static constexpr int kU = kRowBytes / 16;  // 16-byte units per key row
};

// NW waves per block; the first RP / 32 of them own a row tile each, the
// others only help to stage K.
template <int DT, int D, int NW>
__global__ __launch_bounds__(64 * NW) void score_kernel(const typename Elem<DT>::T* __restrict__ K,
                                                        const int32_t* __restrict__ len, int Hkv, int Lmax,
                                                        const typename Elem<DT>::T* __restrict__ obs,
                                                        const int32_t* __restrict__ obs_valid, int RP,
                                                        float* __restrict__ scores, float* __restrict__ lse_out,
                                                        int32_t* __restrict__ ws_words) {
  using Lay = ScoreLayout<DT, D>;
  using MF = Mfma<DT, D>;
  using Frag = typename MF::Frag;
  constexpr int KS = MF::kSteps;
  constexpr int kU = Lay::kU;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* ktile = smem;                                                    // [kTile][kRowStride]
  float* part = reinterpret_cast<float*>(smem + kTile * Lay::kRowStride);          // [NW][kTile]
  float* lse_lds = part + NW * kTile;                                              // [RP]
  const int nrow_waves = RP / 32;

  const size_t unit = blockIdx.x;
  const int n = (int)(unit / Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool has_rows = wave < nrow_waves;
  const int L = len[n];
  if (L < 0 || L > Lmax) {
    if (tid == 0) set_status(ws_words, BKV_DEV_BAD_LEN);
    return;
  }
  if (L == 0) return;

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(K + unit * (size_t)Lmax * D);
  const float scale2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
  const float ninf = -__builtin_huge_valf();

  // query fragment of this wave's 32 rows (lane's row = 32 wave + lane % 32)
  const int myrow = 32 * wave + (lane & 31);
  Frag qf[KS];
  bool row_valid = false;
  if (has_rows) {
    const unsigned char* qrow =
        reinterpret_cast<const unsigned char*>(obs + (unit * RP + myrow) * (size_t)D);
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = MF::load(qrow, s, lane);
    row_valid = obs_valid[unit * RP + myrow] != 0;
  }

  const int ntiles = (L + kTile - 1) / kTile;
  constexpr int nthreads = 64 * NW;
  constexpr int units_per_tile = kTile * kU;
  constexpr int kPerThreadMax = (units_per_tile + nthreads - 1) / nthreads;

  // register prefetch of one tile: thread handles units tid, tid + nthreads, ...
  uint4 pre[kPerThreadMax];
  auto prefetch = [&](int tile) {
    const int key0 = tile * kTile;
#pragma unroll
    for (int k = 0; k < kPerThreadMax; ++k) {
      const int u = tid + k * nthreads;
      if (u < units_per_tile) {
        const int r = u / kU, q = u % kU;
        if (key0 + r < L) {
          pre[k] = reinterpret_cast<const uint4*>(kbase + (size_t)(key0 + r) * Lay::kRowBytes)[q];
        } else {
          pre[k] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int k = 0; k < kPerThreadMax; ++k) {
      const int u = tid + k * nthreads;
      if (u < units_per_tile) {
        const int r = u / kU, q = u % kU;
        reinterpret_cast<uint4*>(ktile + (size_t)r * Lay::kRowStride)[q] = pre[k];
      }
    }
  };

  // ---------------- pass 1: per-row log2-sum-exp ----------------
  float run_m = ninf, run_s = 0.0f;
  prefetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // previous tile fully consumed
    commit();
    __syncthreads();
    if (tile + 1 < ntiles) prefetch(tile + 1);
    const int key0 = tile * kTile;
#pragma unroll
    for (int sub = 0; sub < kTile / kSub; ++sub) {
      if (!has_rows || key0 + sub * kSub >= L) break;
      const unsigned char* krow = ktile + (size_t)(sub * kSub + (lane & 31)) * Lay::kRowStride;
      floatx16_t acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = MF::mma(MF::load(krow, s, lane), qf[s], acc);
      // acc[r]: key sub*32 + acc_row(r, lane), row = lane % 32
      float v[16];
      float mx = ninf;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = key0 + sub * kSub + acc_row(r, lane);
        v[r] = (j < L) ? acc[r] * scale2 : ninf;
        mx = fmaxf(mx, v[r]);
      }
      const float m_new = fmaxf(run_m, mx);
      if (m_new != ninf) {
        float sum = 0.0f;
#pragma unroll
        for (int r = 0; r < 16; ++r) sum += exp2f(v[r] - m_new);
        run_s = run_s * exp2f(run_m - m_new) + sum;
        run_m = m_new;
      }
    }
  }
  // merge the two lanes that hold the same row (lane, lane ^ 32)
  {
    const float om = __shfl_xor(run_m, 32, 64);
    const float os = __shfl_xor(run_s, 32, 64);
    const float m = fmaxf(run_m, om);
    float s = 0.0f;
    if (run_m != ninf) s += run_s * exp2f(run_m - m);
    if (om != ninf) s += os * exp2f(om - m);
    const float lse2 = row_valid ? m + log2f(s) : __builtin_huge_valf();
    if (has_rows && lane < 32) {
      lse_lds[myrow] = lse2;
      lse_out[unit * RP + myrow] = row_valid ? lse2 * 0.69314718055994531f : __builtin_huge_valf();
    }
  }
  __syncthreads();
  // pass 2 orientation: lane = key, acc[r] = row 32 wave + acc_row(r, lane)
  float lse_r[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) lse_r[r] = has_rows ? lse_lds[32 * wave + acc_row(r, lane)] : 0.0f;

  // ---------------- pass 2: per-key max of (s - lse) ----------------
  float* out = scores + unit * (size_t)Lmax;
  prefetch(ntiles - 1);
  for (int tile = ntiles - 1; tile >= 0; --tile) {
    __syncthreads();
    commit();
    __syncthreads();
    if (tile > 0) prefetch(tile - 1);
    const int key0 = tile * kTile;
#pragma unroll
    for (int sub = 0; sub < kTile / kSub; ++sub) {
      if (!has_rows || key0 + sub * kSub >= L) break;
      const unsigned char* krow = ktile + (size_t)(sub * kSub + (lane & 31)) * Lay::kRowStride;
      floatx16_t acc = {};
#pragma unroll
      for (int s = 0; s < KS; ++s) acc = MF::mma(qf[s], MF::load(krow, s, lane), acc);
      float t = ninf;
#pragma unroll
      for (int r = 0; r < 16; ++r) t = fmaxf(t, acc[r] * scale2 - lse_r[r]);
      t = fmaxf(t, __shfl_xor(t, 32, 64));
      if (lane < 32) part[wave * kTile + sub * kSub + lane] = t;
    }
    __syncthreads();
    for (int k = tid; k < kTile; k += nthreads) {
      const int j = key0 + k;
      if (j < L) {
        float t = part[k];
        for (int w = 1; w < nrow_waves; ++w) t = fmaxf(t, part[w * kTile + k]);
        out[j] = exp2f(t);  // exp2(-inf) = 0 when no row is present
      }
    }
  }
}

template <int DT, int D, int NW>
static hipError_t launch_score_nw(const void* K, const int32_t* len, int N, int Hkv, int Lmax, const void* obs,
                                  const int32_t* obs_valid, int RP, float* scores, float* lse, int32_t* ws_words,
                                  hipStream_t st) {
  using Lay = ScoreLayout<DT, D>;
  using ET = typename Elem<DT>::T;
  const size_t smem = (size_t)kTile * Lay::kRowStride + (size_t)NW * kTile * sizeof(float) + RP * sizeof(float);
  auto kern = score_kernel<DT, D, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(N * Hkv), dim3(64 * NW), smem, st, (const ET*)K, len, Hkv, Lmax, (const ET*)obs,
                     obs_valid, RP, scores, lse, ws_words);
  return hipGetLastError();
}

// RP (observation rows rounded up to 32) is at most 256: 1..8 row tiles.
template <int DT, int D>
hipError_t launch_score(const void* K, const int32_t* len, int N, int Hkv, int Lmax, const void* obs,
                        const int32_t* obs_valid, int RP, float* scores, float* lse, int32_t* ws_words,
                        hipStream_t st) {
  const int tiles = RP / 32;
  if (tiles <= 2) return launch_score_nw<DT, D, 2>(K, len, N, Hkv, Lmax, obs, obs_valid, RP, scores, lse, ws_words, st);
  if (tiles <= 4) return launch_score_nw<DT, D, 4>(K, len, N, Hkv, Lmax, obs, obs_valid, RP, scores, lse, ws_words, st);
  return launch_score_nw<DT, D, 8>(K, len, N, Hkv, Lmax, obs, obs_valid, RP, scores, lse, ws_words, st);
}

#define BKV_INST_SCORE(DT, D)                                                                                   \
  template hipError_t launch_score<DT, D>(const void*, const int32_t*, int, int, int, const void*,             \
                                          const int32_t*, int, float*, float*, int32_t*, hipStream_t);
BKV_INST_SCORE(BKV_F32, 64)
BKV_INST_SCORE(BKV_F32, 128)
BKV_INST_SCORE(BKV_BF16, 64)
BKV_INST_SCORE(BKV_BF16, 128)

}  // namespace bkv

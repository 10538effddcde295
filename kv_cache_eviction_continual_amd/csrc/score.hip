// score.hip -- beacon-guided importance scores on gfx950 matrix cores.
//
// For one (slot, KV head) the observation rows are the recent queries and
// beacons of the G query heads of the group.  Each row r attends to every
// cached key:
//   p_r(j) = softmax_j(q_r . k_j / sqrt(d)),  score_j = max_r p_r(j)
// (inkeast.github.io MessageDaily paper-reading post on BeaconKV, sections 三
// and 4.4: scoring by the attention of recent queries together with the
// beacon set; wzjinhao.cn news article 56682, section 信标查询怎么用:
// beacons placed at the current position, recent queries at their own, and
// aggregation by maximum).
//
// rope_table_kernel: per slot, (cos, sin) of every recent position and of
// the current position, one entry per rotated pair.
//
// score_kernel: one workgroup per (slot, KV head), one wave per 32-row tile
// of observation rows.  The wave loads its rows (recent queries, or the
// buffer rows the beacon FPS picked) straight into matrix-core fragments and
// rotates them there: a lane holds dims i and i + d/2 of its row in the same
// element of two fragments.  The rotated rows are written to the workspace
// (a debug copy) and stay in registers for the whole kernel.  K streams
// through LDS in tiles of kTile keys (coalesced 16-byte loads, the next tile
// prefetched into registers while the current one is multiplied).  Two
// passes over K:
//   pass 1: S^T = K Q^T on MFMA (lane = row, 16 keys per lane), online
//           row max and sum of exp2 -> per-row log2-sum-exp; in a full tile
//           the next sub-tile's products are issued among the current one's
//           exp work, so one wave keeps the matrix core and the VALU busy;
//   pass 2: S = Q K^T on MFMA (lane = key, 16 rows per lane), the
//           accumulators starting at -lse_r / scale (so the products land on
//           s - lse_r / scale), per-key max over the wave's rows, then over
//           the waves through LDS; one exp2 per key.  Pass 2 walks the tiles
//           in reverse so that the most recently read tiles are still cached.
// exp(max_r(s_r - lse_r)) = max_r exp(s_r - lse_r), so one exp per key
// suffices.  Logits are accumulated in fp32 from exact bf16 (or fp32)
// products.  The mean-aggregation variant (the same post, section 4.4: max
// or mean) sums exp2(s - lse) over the rows in pass 2 instead and divides by
// the rows present.
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
  using Raw = uint4;  // the same 8 elements as storage bits
  static constexpr int kSteps = D / 16;
  __device__ static inline Raw load_raw(const unsigned char* row, int s, int lane) {
    return *reinterpret_cast<const uint4*>(row + (size_t)(16 * s + 8 * (lane >> 5)) * 2);
  }
  __device__ static inline void store_raw(unsigned char* row, int s, int lane, Raw v) {
    *reinterpret_cast<uint4*>(row + (size_t)(16 * s + 8 * (lane >> 5)) * 2) = v;
  }
  __device__ static inline Raw zero_raw() { return make_uint4(0u, 0u, 0u, 0u); }
  __device__ static inline Frag frag(Raw v) { return __builtin_bit_cast(Frag, v); }
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
  using Raw = float;
  static constexpr int kSteps = D / 2;
  __device__ static inline Raw load_raw(const unsigned char* row, int s, int lane) {
    return *reinterpret_cast<const float*>(row + (size_t)(2 * s + (lane >> 5)) * 4);
  }
  __device__ static inline void store_raw(unsigned char* row, int s, int lane, Raw v) {
    *reinterpret_cast<float*>(row + (size_t)(2 * s + (lane >> 5)) * 4) = v;
  }
  __device__ static inline Raw zero_raw() { return 0.0f; }
  __device__ static inline Frag frag(Raw v) { return v; }
  // dim of lane `lane` at k-step s: 2 s + lane / 32
  __device__ static inline Frag load(const unsigned char* row, int s, int lane) {
    return *reinterpret_cast<const float*>(row + (size_t)(2 * s + (lane >> 5)) * 4);
  }
  __device__ static inline floatx16_t mma(Frag a, Frag b, floatx16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Scheduling pattern for one 32x32 sub-tile's eight products (each with
// its LDS fragment reads) issued among the vector work of the previous
// sub-tile: a product occupies the matrix core for 32 cycles, long enough
// for about six vector instructions of the same wave.
__device__ inline void interleave_products_with_valu() {
  constexpr int kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;
  __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
  __builtin_amdgcn_sched_group_barrier(kValu, 4, 0);
#define BKV_MFMA_THEN_VALU(nds)                           \
  __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);      \
  __builtin_amdgcn_sched_group_barrier(kValu, 6, 0);      \
  __builtin_amdgcn_sched_group_barrier(kDsRead, nds, 0);
  BKV_MFMA_THEN_VALU(2)
  BKV_MFMA_THEN_VALU(0)
  BKV_MFMA_THEN_VALU(2)
  BKV_MFMA_THEN_VALU(0)
  BKV_MFMA_THEN_VALU(2)
  BKV_MFMA_THEN_VALU(0)
  BKV_MFMA_THEN_VALU(0)
  BKV_MFMA_THEN_VALU(0)
#undef BKV_MFMA_THEN_VALU
}

// Accumulator element r of lane l holds output row 8 (r / 4) + 4 (l / 32) +
// r % 4 and output column l % 32 (32x32 MFMA family, checked on gfx950).
__device__ inline int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// RoPE (rotate-half: dim i pairs with dim i + d/2, i < d/2)
// ---------------------------------------------------------------------------

// tab[n][r][i] = (cos, sin) of the angle of pair i at recent position r
// (r < R) or at pos_now (r = R); positions below zero give (1, 0).
template <int D>
__global__ void rope_table_kernel(const int32_t* __restrict__ recent_pos, const int32_t* __restrict__ pos_now,
                                  int R, double theta, float2* __restrict__ tab) {
  const int n = blockIdx.x;
  constexpr int H = D / 2;
  float2* out = tab + (size_t)n * (R + 1) * H;
  for (int e = threadIdx.x; e < (R + 1) * H; e += blockDim.x) {
    const int r = e / H, i = e % H;
    const int pos = r < R ? recent_pos[(size_t)n * R + r] : pos_now[n];
    float2 cs = make_float2(1.0f, 0.0f);
    if (pos >= 0) {
      // inverse frequency theta^(-2i/d) held in binary32; the angle pos * freq
      // is exact in binary64; cos and sin are evaluated in binary64 and held
      // in binary32
      const double freq = (double)(float)pow(theta, -(2.0 * i) / (double)D);
      const double a = (double)pos * freq;
      cs = make_float2((float)cos(a), (float)sin(a));
    }
    out[e] = cs;
  }
}

// One rotated pair: binary64 products of a storage value and a binary32
// cos/sin are exact, so each output is the correctly rounded binary64 value
// of the exact rotation, rounded once more to the storage type.
template <int DT>
__device__ inline void rope_pair(double xa, double xb, float2 cs, typename Elem<DT>::T* ya,
                                 typename Elem<DT>::T* yb) {
  const double c = (double)cs.x, sn = (double)cs.y;
  *ya = Elem<DT>::from_f64(xa * c - xb * sn);
  *yb = Elem<DT>::from_f64(xb * c + xa * sn);
}

// Rotates the fragments of one lane in place.  Fragment s and fragment
// s + kSteps/2 hold the same dims of the two halves of the row.
template <int DT, int D>
struct RopeFrag;

template <int D>
struct RopeFrag<BKV_BF16, D> {
  static constexpr int KS = D / 16;
  // dims of fragment s: 16 s + 8 h + [0, 8), h = lane / 32
  __device__ static inline void rotate(uint4 (&x)[KS], const float2* cs_row, int h) {
#pragma unroll
    for (int s = 0; s < KS / 2; ++s) {
      const float4* c4 = reinterpret_cast<const float4*>(cs_row + 16 * s + 8 * h);
      const float4 c01 = c4[0], c23 = c4[1], c45 = c4[2], c67 = c4[3];
      const float2 cs[8] = {make_float2(c01.x, c01.y), make_float2(c01.z, c01.w), make_float2(c23.x, c23.y),
                            make_float2(c23.z, c23.w), make_float2(c45.x, c45.y), make_float2(c45.z, c45.w),
                            make_float2(c67.x, c67.y), make_float2(c67.z, c67.w)};
      const uint32_t lo[4] = {x[s].x, x[s].y, x[s].z, x[s].w};
      const uint32_t hi[4] = {x[s + KS / 2].x, x[s + KS / 2].y, x[s + KS / 2].z, x[s + KS / 2].w};
      uint32_t ylo[4], yhi[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint16_t a0, a1, b0, b1;
        rope_pair<BKV_BF16>(Elem<BKV_BF16>::to_f64((uint16_t)(lo[w] & 0xFFFF)),
                            Elem<BKV_BF16>::to_f64((uint16_t)(hi[w] & 0xFFFF)), cs[2 * w], &a0, &b0);
        rope_pair<BKV_BF16>(Elem<BKV_BF16>::to_f64((uint16_t)(lo[w] >> 16)),
                            Elem<BKV_BF16>::to_f64((uint16_t)(hi[w] >> 16)), cs[2 * w + 1], &a1, &b1);
        ylo[w] = (uint32_t)a0 | ((uint32_t)a1 << 16);
        yhi[w] = (uint32_t)b0 | ((uint32_t)b1 << 16);
      }
      x[s] = make_uint4(ylo[0], ylo[1], ylo[2], ylo[3]);
      x[s + KS / 2] = make_uint4(yhi[0], yhi[1], yhi[2], yhi[3]);
      __builtin_amdgcn_sched_barrier(0);  // one fragment pair at a time (register pressure)
    }
  }
};

template <int D>
struct RopeFrag<BKV_F32, D> {
  static constexpr int KS = D / 2;
  // dim of fragment s: 2 s + h
  __device__ static inline void rotate(float (&x)[KS], const float2* cs_row, int h) {
#pragma unroll
    for (int s = 0; s < KS / 2; ++s) {
      float a, b;
      rope_pair<BKV_F32>((double)x[s], (double)x[s + KS / 2], cs_row[2 * s + h], &a, &b);
      x[s] = a;
      x[s + KS / 2] = b;
    }
  }
};

template <int DT, int D>
struct ScoreLayout {
  static constexpr int kRowBytes = D * Elem<DT>::kBytes;
  static constexpr int kRowStride = kRowBytes + 16;
  static constexpr int kU = kRowBytes / 16;  // 16-byte units per key row
};

// Waves per SIMD the registers of a NW-wave block are budgeted for: three
// blocks per CU for rows of at most 256 bytes, two for two-wave blocks (each
// lane stages twice as much of a tile); wider (binary32, d = 128) rows take
// what their fragments need.
template <int DT, int D, int NW>
constexpr int score_waves_per_simd() {
  return ScoreLayout<DT, D>::kRowBytes > 256 ? 1 : NW == 2 ? 2 : 3;
}

// NW waves per block; the first RP / 32 of them own a row tile each, the
// others only help to stage K.  Observation row r of the unit is, for
// g = r / (R + nb) and k = r % (R + nb): recent query k of query head
// h G + g (present if its position is >= 0), or for k >= R its beacon k - R
// (present if below the pick count; read from the picks kernel's row copy);
// rows from G (R + nb) to RP are padding.
template <int DT, int D, int NW, bool kMean>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(score_waves_per_simd<DT, D, NW>()))) void score_kernel(
    const typename Elem<DT>::T* __restrict__ K, const int32_t* __restrict__ len, int Hkv, int Hq, int Lmax,
    const typename Elem<DT>::T* __restrict__ recent, const int32_t* __restrict__ recent_pos, int R,
    const int32_t* __restrict__ beacons, const typename Elem<DT>::T* __restrict__ brows, int nb,
    const float2* __restrict__ tab, typename Elem<DT>::T* __restrict__ obs, int32_t* __restrict__ obs_valid, int RP,
    float* __restrict__ scores, float* __restrict__ lse_out, const float* __restrict__ capture,
    int32_t* __restrict__ ws_words) {
  using Lay = ScoreLayout<DT, D>;
  using MF = Mfma<DT, D>;
  using Frag = typename MF::Frag;
  using Raw = typename MF::Raw;
  constexpr int KS = MF::kSteps;
  constexpr int kU = Lay::kU;
  constexpr int H = D / 2;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* ktile = smem;                                                    // [kTile][kRowStride]
  float* part = reinterpret_cast<float*>(smem + kTile * Lay::kRowStride);          // [NW][kTile]
  float* lse_lds = part + NW * kTile;                                              // [RP]
  int* nvalid_lds = reinterpret_cast<int*>(lse_lds + RP);                          // [NW] present rows per wave
  const int nrow_waves = RP / 32;

  const size_t unit = blockIdx.x;
  const int n = (int)(unit / Hkv);
  const int hkv = (int)(unit % Hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool has_rows = wave < nrow_waves;
  const int L = len[n];
  if (L < 0 || L > Lmax) {
    if (tid == 0) set_status(ws_words, BKV_DEV_BAD_LEN);
    return;
  }

  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(K + unit * (size_t)Lmax * D);
  const float scale2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)
  const float ninf = -__builtin_huge_valf();

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

  // the first K tile is in flight while the rows are built
  if (L > 0) prefetch(0);

  // this lane's observation row (two lanes per row, h = lane / 32): load it
  // into fragments, rotate it, keep it, and write the debug copy
  const int myrow = 32 * wave + (lane & 31);
  Frag qf[KS];
  bool row_valid = false;
  if (has_rows) {
    const int G = Hq / Hkv;
    const int per = R + nb;  // > 0 whenever RP > 0
    const int g = min(myrow / per, G - 1);
    const int k = myrow - (myrow / per) * per;
    const size_t head = (size_t)n * Hq + (size_t)hkv * G + g;
    const int32_t* bk = beacons + head * (nb + 1);
    const unsigned char* src;
    if (k < R) {
      row_valid = recent_pos[(size_t)n * R + k] >= 0;
      src = reinterpret_cast<const unsigned char*>(recent + (head * R + k) * D);
    } else {  // beacon k - R: the picks kernel's copy of its buffer row
      row_valid = k - R < bk[0];
      src = reinterpret_cast<const unsigned char*>(brows + (head * nb + (row_valid ? k - R : 0)) * D);
    }
    row_valid = row_valid && myrow < G * per;
    Raw x[KS];
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) x[s2] = MF::load_raw(src, s2, lane);
    RopeFrag<DT, D>::rotate(x, tab + ((size_t)n * (R + 1) + (k < R ? k : R)) * H, lane >> 5);
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      if (!row_valid) x[s2] = MF::zero_raw();
      qf[s2] = MF::frag(x[s2]);
    }
    if (obs != nullptr) {  // the debug copy of the rotated rows
      unsigned char* orow = reinterpret_cast<unsigned char*>(obs + (unit * RP + myrow) * (size_t)D);
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) MF::store_raw(orow, s2, lane, x[s2]);
    }
    if (lane < 32) obs_valid[unit * RP + myrow] = row_valid ? 1 : 0;
  }
  if constexpr (kMean) {
    const uint64_t present = __ballot(has_rows && lane < 32 && row_valid);
    if (lane == 0) nvalid_lds[wave] = __builtin_popcountll(present);
  }
  if (L == 0) {
    if (has_rows && lane < 32) lse_out[unit * RP + myrow] = __builtin_huge_valf();
    return;
  }

  // ---------------- pass 1: per-row log2-sum-exp ----------------
  float run_m = ninf, run_s = 0.0f;
  // S^T for key sub-tile `sub` of the LDS tile: acc[r] is key
  // sub*32 + acc_row(r, lane) of row lane % 32
  auto logits_t = [&](int sub) {
    const unsigned char* krow = ktile + (size_t)(sub * kSub + (lane & 31)) * Lay::kRowStride;
    floatx16_t acc = {};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = MF::mma(MF::load(krow, s, lane), qf[s], acc);
    return acc;
  };
  // every key of the sub-tile present: the scale is positive, so the maximum
  // of the raw logits scales to the maximum of the scaled ones; one fma and
  // one hardware exp2 per key (a term below 2^-126 of the running maximum is
  // flushed to 0, which the sum of at least 1 cannot see)
  auto fold_full = [&](const floatx16_t& acc) {
    float mx = acc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, acc[r]);
    const float m_new = fmaxf(run_m, mx * scale2);
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += __builtin_amdgcn_exp2f(fmaf(acc[r], scale2, -m_new));
    run_s = run_s * __builtin_amdgcn_exp2f(run_m - m_new) + sum;
    run_m = m_new;
  };
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // previous tile fully consumed
    commit();
    __syncthreads();
    if (tile + 1 < ntiles) prefetch(tile + 1);
    const int key0 = tile * kTile;
    if (!has_rows) continue;
    if (key0 + kTile <= L) {
      // a full tile: the products of sub-tile sub + 1 are issued before the
      // exp work of sub-tile sub, so the matrix cores and the vector ALUs of
      // the wave overlap
      floatx16_t cur = logits_t(0);
#pragma unroll
      for (int sub = 0; sub < kTile / kSub; ++sub) {
        floatx16_t next = cur;
        if (sub + 1 < kTile / kSub) next = logits_t(sub + 1);
        fold_full(cur);
        if (sub + 1 < kTile / kSub) interleave_products_with_valu();
        __builtin_amdgcn_sched_barrier(0);  // one sub-tile pair per scheduling region
        cur = next;
      }
      continue;
    }
#pragma unroll
    for (int sub = 0; sub < kTile / kSub; ++sub) {
      if (key0 + sub * kSub >= L) break;
      const floatx16_t acc = logits_t(sub);
      if (key0 + sub * kSub + kSub <= L) {
        fold_full(acc);
      } else {
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
  float inv_present = 0.0f;  // mean aggregation: 1 / (rows present in the unit), 0 if none
  if constexpr (kMean) {
    int present = 0;
    for (int w = 0; w < nrow_waves; ++w) present += nvalid_lds[w];
    inv_present = present > 0 ? 1.0f / (float)present : 0.0f;
  }

  // ---------------- pass 2: per-key max of (s - lse) ----------------
  float* out = scores + unit * (size_t)Lmax;
  // S for key sub-tile `sub`: acc[r] is row 32 wave + acc_row(r, lane) of
  // key sub*32 + lane % 32
  // max aggregation: each accumulator starts at -lse_r / scale2 (-inf for an
  // absent row), so the products land on s - lse_r / scale2 and a key's score
  // exp2(max_r (s scale2 - lse_r)) is exp2(scale2 max_r acc_r): one max per
  // logit, no fma (scale2 > 0 keeps the maximum)
  floatx16_t acc0 = {};
  if constexpr (!kMean) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc0[r] = -lse_r[r] / scale2;
  }
  auto logits = [&](int sub) {
    const unsigned char* krow = ktile + (size_t)(sub * kSub + (lane & 31)) * Lay::kRowStride;
    floatx16_t acc = acc0;
#pragma unroll
    for (int s = 0; s < KS; ++s) acc = MF::mma(qf[s], MF::load(krow, s, lane), acc);
    return acc;
  };
  // the wave's rows folded per key into part[wave][key]
  auto reduce_rows = [&](const floatx16_t& acc, int sub) {
    float t;
    if constexpr (kMean) {  // sum of the rows' probabilities (absent rows: lse +inf, probability 0)
      t = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) t += __builtin_amdgcn_exp2f(fmaf(acc[r], scale2, -lse_r[r]));
      t += __shfl_xor(t, 32, 64);
    } else {  // maximum over the rows of s - lse_r / scale2
      t = acc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) t = fmaxf(t, acc[r]);
      t = fmaxf(t, __shfl_xor(t, 32, 64));
    }
    if (lane < 32) part[wave * kTile + sub * kSub + lane] = t;
  };
  prefetch(ntiles - 1);
  for (int tile = ntiles - 1; tile >= 0; --tile) {
    __syncthreads();
    commit();
    __syncthreads();
    if (tile > 0) prefetch(tile - 1);
    const int key0 = tile * kTile;
    if (has_rows && key0 + kTile <= L) {
      // a full tile: products of sub-tile sub + 1 among the reduction of sub
      floatx16_t cur = logits(0);
#pragma unroll
      for (int sub = 0; sub < kTile / kSub; ++sub) {
        floatx16_t next = cur;
        if (sub + 1 < kTile / kSub) next = logits(sub + 1);
        reduce_rows(cur, sub);
        if (sub + 1 < kTile / kSub) interleave_products_with_valu();
        __builtin_amdgcn_sched_barrier(0);
        cur = next;
      }
    } else if (has_rows) {
#pragma unroll
      for (int sub = 0; sub < kTile / kSub; ++sub) {
        if (key0 + sub * kSub >= L) break;
        reduce_rows(logits(sub), sub);
      }
    }
    __syncthreads();
    for (int k = tid; k < kTile; k += nthreads) {
      const int j = key0 + k;
      if (j < L) {
        float t = part[k];
        if constexpr (kMean) {
          for (int w = 1; w < nrow_waves; ++w) t += part[w * kTile + k];
          out[j] = t * inv_present;
        } else {
          for (int w = 1; w < nrow_waves; ++w) t = fmaxf(t, part[w * kTile + k]);
          float v = exp2f(t * scale2);  // exp2(-inf) = 0 when no row is present
          if (capture != nullptr) v = fmaxf(v, capture[unit * (size_t)Lmax + j]);  // the recent rows' captured maxima
          out[j] = v;
        }
      }
    }
  }
}

template <int DT, int D, int NW, bool kMean>
static hipError_t launch_score_nw(const void* K, const int32_t* len, int N, int Hkv, int Hq, int Lmax,
                                  const void* recent, const int32_t* recent_pos, int R, const int32_t* beacons,
                                  const void* brows, int nb, const float2* tab, void* obs, int32_t* obs_valid,
                                  int RP, float* scores, float* lse, const float* capture, int32_t* ws_words,
                                  hipStream_t st) {
  using Lay = ScoreLayout<DT, D>;
  using ET = typename Elem<DT>::T;
  const size_t smem = (size_t)kTile * Lay::kRowStride + (size_t)NW * kTile * sizeof(float) + RP * sizeof(float) +
                      NW * sizeof(int);
  auto kern = score_kernel<DT, D, NW, kMean>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(N * Hkv), dim3(64 * NW), smem, st, (const ET*)K, len, Hkv, Hq, Lmax,
                     (const ET*)recent, recent_pos, R, beacons, (const ET*)brows, nb, tab, (ET*)obs, obs_valid, RP,
                     scores, lse, capture, ws_words);
  return hipGetLastError();
}

// The RoPE table, then the scores.  RP (observation rows rounded up to 32)
// is at most 256: 1..8 row tiles.
template <int DT, int D>
hipError_t launch_score(const void* K, const int32_t* len, int N, int Hkv, int Hq, int Lmax, const void* recent,
                        const int32_t* recent_pos, int R, const int32_t* beacons, const void* brows, int nb,
                        const int32_t* pos_now, double theta, float2* tab, void* obs, int32_t* obs_valid, int RP,
                        float* scores, float* lse, int32_t* ws_words, bool mean, const float* capture,
                        hipStream_t st) {
  hipLaunchKernelGGL(rope_table_kernel<D>, dim3(N), dim3(256), 0, st, recent_pos, pos_now, R, theta, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int tiles = RP / 32;
#define BKV_SCORE_NW(NW)                                                                                       \
  return mean ? launch_score_nw<DT, D, NW, true>(K, len, N, Hkv, Hq, Lmax, recent, recent_pos, R, beacons, brows, \
                                                 nb, tab, obs, obs_valid, RP, scores, lse, nullptr, ws_words, st) \
              : launch_score_nw<DT, D, NW, false>(K, len, N, Hkv, Hq, Lmax, recent, recent_pos, R, beacons,      \
                                                  brows, nb, tab, obs, obs_valid, RP, scores, lse, capture,      \
                                                  ws_words, st)
  if (tiles <= 2) BKV_SCORE_NW(2);
  if (tiles <= 4) BKV_SCORE_NW(4);
  BKV_SCORE_NW(8);
#undef BKV_SCORE_NW
}

#define BKV_INST_SCORE(DT, D)                                                                                  \
  template hipError_t launch_score<DT, D>(const void*, const int32_t*, int, int, int, int, const void*,       \
                                          const int32_t*, int, const int32_t*, const void*, int,              \
                                          const int32_t*, double, float2*, void*, int32_t*, int, float*,      \
                                          float*, int32_t*, bool, const float*, hipStream_t);
BKV_INST_SCORE(BKV_F32, 64)
BKV_INST_SCORE(BKV_F32, 128)
BKV_INST_SCORE(BKV_BF16, 64)
BKV_INST_SCORE(BKV_BF16, 128)

}  // namespace bkv

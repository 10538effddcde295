// fps.hip -- Continual farthest point sampling on gfx950.
//
// Two kernels share one FPS routine:
//   fps_update_kernel  ingest of new pre-RoPE queries into the bounded
//                      per-query-head buffer, shrinking it by FPS whenever it
//                      fills (wzjinhao.cn news article 56682 on BeaconKV,
//                      section 怎么挑出这几个信标: bounded buffer per head,
//                      FPS compression back to a smaller size when full);
//   beacon_pick_kernel beacon selection by FPS over the live buffer (same
//                      article, section 信标查询怎么用: the beacons are the
//                      FPS representatives of the buffer); the score kernel
//                      rotates the picked rows itself.
//
// FPS on cosine similarity: start at the row with the lowest mean cosine to
// all rows; then repeatedly add the row with the lowest maximum cosine to the
// picked set; ties go to the lower row.
//
// Capacities above 128 rows use a second, cooperative routine (fps_coop):
// one workgroup of eight waves per head, described where it is defined.
//
// One wavefront per query head, no block barriers.  The head's rows stay in
// global memory (they are read once into matrix-core fragments, and again
// only for binary64 decisions and the write-back); LDS holds the packed
// strict lower triangle of the fp32 Gram matrix (32.5 KB for 128 rows, so
// four heads share a CU).
//
// The decisions are those of binary64 evaluation:
//   * squared norms are fp32 sums of exact products (dot2 on bf16), so
//     1/|x| carries a relative error below d u / 2 + 2 u (u = 2^-24); the
//     Gram matrix comes from the matrix cores (exact bf16 products, fp32
//     sums: error below d u |x_i| |x_j|).  Every fp32 cosine
//     G_ij / (|x_i| |x_j|) is therefore within (2 d + 6) u of the exact one,
//     plus at most 2^-19 for products flushed below the fp32 normal range;
//     the decisions use the wider bound eps = 4 (d + 8) u, and the mean
//     cosines eps + 4 (c + 8) u (c-term fp32 sum and one division more);
//   * candidates are compared on keys (order-preserving fp32 bits, low 8
//     bits replaced by the row index).  Every candidate whose fp32 value is
//     within 2 eps of the best key's bucket could hold the true minimum; when
//     there is more than one, they are evaluated from the rows in binary64
//     and the lowest value wins, ties to the lower row;
//   * a row whose squared norm leaves [1e-30, 1e36], or a nonzero row whose
//     fp32 squared norm underflows to 0, sends the whole call to binary64
//     rounds over every candidate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 fps_bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 fps_bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float fps_floatx16;
typedef float fps_float8 __attribute__((ext_vector_type(8)));

constexpr float kFpsU = 5.9604644775390625e-8f;  // 2^-24

// Offset of row i in the packed strict lower triangle (entries (i, j), j < i).
__host__ __device__ constexpr int tri(int i) { return i * (i - 1) / 2; }

// ---------------------------------------------------------------------------
// Matrix-core fragments per storage type
// ---------------------------------------------------------------------------

template <int DT, int D>
struct FpsFrag;

// v_mfma_f32_32x32x16_bf16: lane (n, h) = (lane % 32, lane / 32) supplies
// row n of its 32-row tile, dims 16 ks + 8 h + [0, 8).
template <int D>
struct FpsFrag<BKV_BF16, D> {
  using T = uint16_t;
  using V = uint4;
  static constexpr int kSteps = D / 16;
  __device__ static inline V load(const T* row, int ks, int h) {
    return *reinterpret_cast<const uint4*>(row + 16 * ks + 8 * h);
  }
  __device__ static inline V zero() { return make_uint4(0u, 0u, 0u, 0u); }
  __device__ static inline void store(T* row, int ks, int h, V v) {
    *reinterpret_cast<uint4*>(row + 16 * ks + 8 * h) = v;
  }
  __device__ static inline fps_floatx16 mma(V a, V b, fps_floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(fps_bf16x8, a),
                                                  __builtin_bit_cast(fps_bf16x8, b), c, 0, 0, 0);
  }
  __device__ static inline float sq2(uint32_t w, float acc) {
    const fps_bf16x2 x = __builtin_bit_cast(fps_bf16x2, w);
    return __builtin_amdgcn_fdot2_f32_bf16(x, x, acc, false);
  }
  __device__ static inline float sumsq(V v, float acc) {
    return sq2(v.w, sq2(v.z, sq2(v.y, sq2(v.x, acc))));
  }
  __device__ static inline uint32_t nonzero(V v) { return (v.x | v.y | v.z | v.w) & 0x7FFF7FFFu; }
};

// v_mfma_f32_32x32x2f32: lane (n, h) supplies row n, dim 2 ks + h.
template <int D>
struct FpsFrag<BKV_F32, D> {
  using T = float;
  using V = float;
  static constexpr int kSteps = D / 2;
  __device__ static inline V load(const T* row, int ks, int h) { return row[2 * ks + h]; }
  __device__ static inline V zero() { return 0.0f; }
  __device__ static inline void store(T* row, int ks, int h, V v) { row[2 * ks + h] = v; }
  __device__ static inline fps_floatx16 mma(V a, V b, fps_floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline float sumsq(V v, float acc) { return fmaf(v, v, acc); }
  __device__ static inline uint32_t nonzero(V v) { return __float_as_uint(v) & 0x7FFFFFFFu; }
};

// ---------------------------------------------------------------------------
// Row sources and LDS layout
// ---------------------------------------------------------------------------

// Buffer row r lives at map[r]: values below C are rows of the buffer as it
// was on entry, values C + t are arrival t of the call.
template <int DT, int D>
struct FpsRows {
  const typename Elem<DT>::T* buf;
  const typename Elem<DT>::T* qn;
  const int* map;  // LDS
  int C;
  __device__ inline const typename Elem<DT>::T* row(int r) const {
    const int v = map[r];
    return v < C ? buf + (size_t)v * D : qn + (size_t)(v - C) * D;
  }
};

struct FpsLds {
  float* gram;           // packed strict lower triangle of the Gram matrix
  unsigned char* stage;  // aliases gram: rows staged for the buffer write-back
  float* inv32;          // [cap] fp32 1 / |x| (0 for rows past the count)
  int* map;              // [cap]
  int* picks;            // [cap]
  int* pos;              // [cap] position of a row among the picks, -1 if not picked
};

template <int DT, int D>
__host__ __device__ constexpr size_t fps_gram_bytes(int cap, int M) {
  const size_t g = ((size_t)tri(cap) + 64) * 4;  // + a pad: the greedy may read one entry past the end
  const size_t st = (size_t)M * D * Elem<DT>::kBytes;
  return ((g > st ? g : st) + 15) & ~(size_t)15;
}

template <int DT, int D>
__host__ __device__ constexpr size_t fps_lds_bytes(int cap, int M) {
  return fps_gram_bytes<DT, D>(cap, M) + (size_t)cap * (4 + 4 + 4 + 4);
}

template <int DT, int D>
__device__ inline FpsLds fps_carve(unsigned char* smem, int cap, int M) {
  const size_t gb = fps_gram_bytes<DT, D>(cap, M);
  FpsLds s;
  s.gram = reinterpret_cast<float*>(smem);
  s.stage = smem;
  s.inv32 = reinterpret_cast<float*>(smem + gb);
  s.map = reinterpret_cast<int*>(smem + gb + (size_t)cap * 4);
  s.picks = reinterpret_cast<int*>(smem + gb + (size_t)cap * 8);
  s.pos = reinterpret_cast<int*>(smem + gb + (size_t)cap * 12);
  return s;
}

// ---------------------------------------------------------------------------
// Wave-level helpers
// ---------------------------------------------------------------------------

__device__ inline int fps_lane() { return threadIdx.x & 63; }

__device__ inline double readfirstlane_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Candidate keys: an fp32 value made order-preserving as a uint32, its low 8
// bits replaced by the row index (rows < 256).  The minimum key is the row
// with the lowest value bucket, ties to the lower row; a bucket spans 256
// ulps of the value, which the callers add to their decision window.
__device__ inline uint32_t cand_key(float v, int row) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (ord & 0xFFFFFF00u) | (uint32_t)row;
}
// Lowest value of the bucket after a key's bucket (an upper bound of every
// value in the key's bucket).
__device__ inline float key_hi(uint32_t k) {
  const uint32_t ord = (k | 0xFFu) + 1u;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int N>
__device__ inline uint32_t row_ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xF, 0xF, false);
}

// Smallest key of the wave: rows of 16 lanes reduce by DPP rotation, the
// four rows through scalar lane reads.  The result is wave-uniform.
__device__ inline uint32_t wave_min_key(uint32_t a) {
  a = min(a, row_ror_u<8>(a));
  a = min(a, row_ror_u<4>(a));
  a = min(a, row_ror_u<2>(a));
  a = min(a, row_ror_u<1>(a));
  uint32_t w = (uint32_t)__builtin_amdgcn_readlane((int)a, 0);
  w = min(w, (uint32_t)__builtin_amdgcn_readlane((int)a, 16));
  w = min(w, (uint32_t)__builtin_amdgcn_readlane((int)a, 32));
  w = min(w, (uint32_t)__builtin_amdgcn_readlane((int)a, 48));
  return w;
}

// ---------------------------------------------------------------------------
// Binary64 decisions
// ---------------------------------------------------------------------------

// binary64 a.b, a.a and b.b of two rows; each row's loads go out together
// (up to 8 units of 16 bytes at a time) before the arithmetic
template <int DT, int D, int kBatch = 8>
__device__ inline void fps_dots64(const typename Elem<DT>::T* a, const typename Elem<DT>::T* b, double& ab,
                                  double& aa, double& bb) {
  using E = Elem<DT>;
  constexpr int kPer16 = 16 / E::kBytes;
  constexpr int kU = D / kPer16;
  constexpr int kC = kU < kBatch ? kU : kBatch;
  const uint4* xa = reinterpret_cast<const uint4*>(a);
  const uint4* xb = reinterpret_cast<const uint4*>(b);
  ab = aa = bb = 0.0;
#pragma unroll
  for (int u0 = 0; u0 < kU; u0 += kC) {
    uint4 wa[kC], wb[kC];
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      wa[u] = xa[u0 + u];
      wb[u] = xb[u0 + u];
    }
#pragma unroll
    for (int u = 0; u < kC; ++u) {
      const typename E::T* ea = reinterpret_cast<const typename E::T*>(&wa[u]);
      const typename E::T* eb = reinterpret_cast<const typename E::T*>(&wb[u]);
#pragma unroll
      for (int k = 0; k < kPer16; ++k) {
        const double va = E::to_f64(ea[k]), vb = E::to_f64(eb[k]);
        ab = fma(va, vb, ab);
        aa = fma(va, va, aa);
        bb = fma(vb, vb, bb);
      }
      // keep the binary64 conversions of one unit at a time in registers
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Lowest binary64 objective among the candidates flagged in `inmask` (bit b
// of word w = row 64 w + b, at least one set), ties to the lower row; a
// flagged row in every case (with NaN objectives, from non-finite rows, the
// lowest flagged row that no finite objective beats).  Objective: the mean
// cosine to all c rows (sum_mode) or the maximum cosine to picks[0, npicked),
// cosines as a.b / (max(|a|, 1e-12) max(|b|, 1e-12)).  The lanes split the
// partner rows; the result is wave-uniform.
template <int DT, int D, int SL, class LdsT, int kBatch = 8>
__device__ __attribute__((always_inline)) int fps_exact_argmin(const FpsRows<DT, D>& src, const LdsT& s,
                                                               const uint64_t* inmask, int c, int npicked,
                                                               bool sum_mode) {
  const int lane = fps_lane();
  const int npart = sum_mode ? c : npicked;
  const double inf = __builtin_huge_val();
  double best = inf;
  int besti = 0x7fffffff;
#pragma unroll
  for (int w = 0; w < SL; ++w) {
    uint64_t m = inmask[w];
    while (m) {
      const int a = 64 * w + (int)__builtin_ctzll(m);
      m &= m - 1;
      const typename Elem<DT>::T* xa = src.row(a);
      double acc = sum_mode ? 0.0 : -inf;
#pragma unroll 1
      for (int q = lane; q < npart; q += 64) {
        const int b = sum_mode ? q : s.picks[q];
        double ab, aa, bb;
        fps_dots64<DT, D, kBatch>(xa, src.row(b), ab, aa, bb);
        const double na = sqrt(aa), nb = sqrt(bb);
        const double v = ab * (1.0 / (na < 1e-12 ? 1e-12 : na)) * (1.0 / (nb < 1e-12 ? 1e-12 : nb));
        acc = sum_mode ? acc + v : fmax(acc, v);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const double o = __shfl_xor(acc, off, 64);
        acc = sum_mode ? acc + o : fmax(acc, o);
      }
      const double obj = readfirstlane_f64(sum_mode ? acc / (double)c : acc);
      // candidates come in increasing row order: ties keep the lower row.  The
      // first candidate is always taken, so the result is a flagged row even
      // when non-finite rows make every objective NaN
      if (obj < best || besti == 0x7fffffff) {
        best = obj;
        besti = a;
      }
    }
  }
  return besti;
}

// ---------------------------------------------------------------------------
// FPS of one head by one wavefront
// ---------------------------------------------------------------------------

// Whether fps_wave keeps every row's matrix-core fragments in registers (at
// most 128 of them per lane) rather than reloading them per use.
template <int DT, int D, int NT>
__host__ __device__ constexpr bool fps_holds() {
  return NT * FpsFrag<DT, D>::kSteps * (int)(sizeof(typename FpsFrag<DT, D>::V) / 4) <= 128;
}

// Rows of the picks written to wb + i d (pick i) straight from the matrix-core
// fragments of their owner lanes (lane (n, h) holds half of row 32 t + n of
// every tile t).  No-op when wb is null.
template <int DT, int D, int NT>
__device__ __forceinline__ void fps_write_picks(const FpsLds& s, int kk,
                                                const typename FpsFrag<DT, D>::V (&fr)[NT][FpsFrag<DT, D>::kSteps],
                                                typename Elem<DT>::T* wb, int lane) {
  using FR = FpsFrag<DT, D>;
  if (wb == nullptr) return;
  const int n = lane & 31, h = lane >> 5;
  for (int r = lane; r < 32 * NT; r += 64) s.pos[r] = -1;
  __builtin_amdgcn_wave_barrier();
  for (int i = lane; i < kk; i += 64) s.pos[s.picks[i]] = i;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = s.pos[32 * t + n];
    if (i >= 0) {
#pragma unroll
      for (int ks = 0; ks < FR::kSteps; ++ks) FR::store(wb + (size_t)i * D, ks, h, fr[t][ks]);
    }
  }
}

// Writes the FPS picks of rows [0, c) (c <= 32 NT) to s.picks, min(k, c) of
// them, and returns the count.  When `wb` is given and the fragments are held
// in registers, also writes pick i's row to wb + i d straight from them.
// Every lane of the wave must call it.
template <int DT, int D, int NT>
__device__ __attribute__((always_inline)) int fps_wave(const FpsRows<DT, D>& src, const FpsLds& s, int c, int k,
                                                       typename Elem<DT>::T* wb = nullptr) {
  using FR = FpsFrag<DT, D>;
  using V = typename FR::V;
  using T = typename Elem<DT>::T;
  constexpr int KS = FR::kSteps;
  constexpr int SL = (NT + 1) / 2;  // candidate slots per lane: rows lane + 64 sl
  constexpr float kEps = 4.0f * (D + 8) * kFpsU;
  const int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  // the lane id passes through an empty asm statement, so the many
  // lane-derived addresses below are computed where they are used rather
  // than hoisted out of a caller's loop and held in registers
  int lane = fps_lane();
  __asm__ volatile("" : "+v"(lane));
  const int n = lane & 31, h = lane >> 5;
  const float finf = __builtin_huge_valf();

  // 1. matrix-core fragments of every row (rows past the count are zero),
  // held in registers when they fit in 128 of them, else reloaded per use
  constexpr bool kHold = fps_holds<DT, D, NT>();
  const T* rowp[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) rowp[t] = 32 * t + n < c ? src.row(32 * t + n) : nullptr;
  auto frag = [&](int t, int ks) -> V { return rowp[t] ? FR::load(rowp[t], ks, h) : FR::zero(); };
  V fr[kHold ? NT : 1][kHold ? KS : 1];
  if constexpr (kHold) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) fr[t][ks] = frag(t, ks);
    }
  }

  // 2. fp32 inverse norms; lane (n, h) keeps those of rows 32 t + n (vector
  // types: per-lane selections below must not turn into indexed memory)
  fps_float8 invr = {};
  int unsafe = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float ss = 0.0f;
    uint32_t nz = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      V v;
      if constexpr (kHold) v = fr[t][ks];
      else v = frag(t, ks);
      ss = FR::sumsq(v, ss);
      nz |= FR::nonzero(v);
    }
    ss += __shfl_xor(ss, 32, 64);
    nz |= (uint32_t)__shfl_xor((int)nz, 32, 64);
    const int r = 32 * t + n;
    float inv = 0.0f;
    if (r < c) {
      if (ss > 0.0f) {
        if (!(ss >= 1e-30f && ss <= 1e36f)) unsafe = 1;
        inv = (float)(1.0 / sqrt((double)ss));
      } else {
        if (nz) unsafe = 1;  // nonzero row whose fp32 squares underflow
        inv = 1e12f;         // zero row: norm clamped at 1e-12, every cosine 0
      }
    }
    invr[t] = inv;
    if (h == 0) s.inv32[r] = inv;
  }
  uint64_t valid[SL];
#pragma unroll
  for (int w = 0; w < SL; ++w) {
    const int cnt = c - 64 * w;
    valid[w] = cnt >= 64 ? ~0ull : (cnt > 0 ? ((1ull << cnt) - 1) : 0ull);
  }
  __builtin_amdgcn_wave_barrier();

  if (__ballot(unsafe) != 0) {  // binary64 rounds over every candidate
    uint64_t avail[SL];
#pragma unroll
    for (int w = 0; w < SL; ++w) avail[w] = valid[w];
    for (int t = 0; t < kk; ++t) {
      const int pick = fps_exact_argmin<DT, D, SL>(src, s, avail, c, t, t == 0);
#pragma unroll
      for (int w = 0; w < SL; ++w)
        if ((pick >> 6) == w) avail[w] &= ~(1ull << (pick & 63));
      if (lane == 0) s.picks[t] = pick;
      __builtin_amdgcn_wave_barrier();
    }
    if constexpr (kHold) fps_write_picks<DT, D, NT>(s, kk, fr, wb, lane);
    return kk;
  }

  // 3. Gram matrix on the matrix cores, one 32-row tile at a time (the MFMA
  // chain is straight-line code): column sums of G_ij / |x_i| for the mean
  // cosines, and the strict lower triangle into LDS
  fps_float8 cs = {};
  const int pad = tri(32 * NT) + lane;  // per-lane slot in the LDS pad past the triangle
#pragma unroll
  for (int tr = 0; tr < NT; ++tr) {
    fps_floatx16 acc[NT];
#pragma unroll
    for (int tc = 0; tc < NT; ++tc) acc[tc] = fps_floatx16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (kHold) {
#pragma unroll
        for (int tc = 0; tc < NT; ++tc) acc[tc] = FR::mma(fr[tr][ks], fr[tc][ks], acc[tc]);
      } else {
        const V a = frag(tr, ks);
#pragma unroll
        for (int tc = 0; tc < NT; ++tc) acc[tc] = FR::mma(a, frag(tc, ks), acc[tc]);
      }
    }
    // accumulator r of lane (n, h) holds G(32 tr + 8 (r / 4) + 4 h + r % 4, 32 tc + n)
    const float4* ivp = reinterpret_cast<const float4*>(s.inv32 + 32 * tr + 4 * h);
    const float4 iv[4] = {ivp[0], ivp[2], ivp[4], ivp[6]};
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i0 = 32 * tr + 8 * (r >> 2) + (r & 3);  // row for h = 0; i = i0 + 4 h
      const int rowoff = tri(i0) + (h ? 4 * i0 + 6 : 0) + n;  // tri(i) + n
      const float4 q = iv[r >> 2];
      const float w = (r & 3) == 0 ? q.x : (r & 3) == 1 ? q.y : (r & 3) == 2 ? q.z : q.w;
#pragma unroll
      for (int tc = 0; tc < NT; ++tc) {
        const float g = acc[tc][r];
        cs[tc] = fmaf(g, w, cs[tc]);
        if (tr > tc) {
          s.gram[rowoff + 32 * tc] = g;
        } else if (tr == tc) {  // strict lower half of a diagonal tile; the rest goes to a pad slot
          s.gram[i0 + 4 * h > 32 * tc + n ? rowoff + 32 * tc : pad] = g;
        }
      }
    }
  }
  fps_float8 S = {};
#pragma unroll
  for (int tc = 0; tc < NT; ++tc) S[tc] = cs[tc] + __shfl_xor(cs[tc], 32, 64);

  // candidate slots of this lane: row j = 64 sl + lane = 32 (2 sl + h) + n
  float invj[SL];
  int trij[SL];
#pragma unroll
  for (int w = 0; w < SL; ++w) {
    invj[w] = (2 * w + 1 < NT) ? (h ? invr[2 * w + 1] : invr[2 * w]) : invr[2 * w];
    trij[w] = tri(min(64 * w + lane, c - 1));
  }

  // 4. start: lowest mean cosine
  int pick;
  {
    float mu[SL];
    uint32_t a = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < SL; ++w) {
      const int j = 64 * w + lane;
      const float sj = (2 * w + 1 < NT) ? (h ? S[2 * w + 1] : S[2 * w]) : S[2 * w];
      mu[w] = j < c ? (sj * invj[w]) / (float)c : finf;
      a = min(a, j < c ? cand_key(mu[w], j) : 0xFFFFFFFFu);
    }
    const uint32_t k1 = wave_min_key(a);
    // every candidate within 2 eps of the best one's bucket could be the
    // true minimum: decide in binary64 when there is more than one
    const float eps_mu = kEps + 4.0f * (float)(c + 8) * kFpsU;
    const float hi1 = key_hi(k1) + 2.0f * eps_mu;
    uint64_t inmask[SL];
    int inwin = 0;
#pragma unroll
    for (int w = 0; w < SL; ++w) {
      inmask[w] = __ballot(64 * w + lane < c && mu[w] <= hi1);
      inwin += __builtin_popcountll(inmask[w]);
    }
    if (inwin > 1) {
      pick = fps_exact_argmin<DT, D, SL>(src, s, inmask, c, 0, true);
    } else {
      pick = (int)(k1 & 0xFFu);
    }
  }
  if (lane == 0) s.picks[0] = pick;

  // 5. greedy rounds on fp32 cosines with the certified window
  const float eps2 = 2.0f * kEps;
  float mt[SL];
  bool picked[SL];
#pragma unroll
  for (int w = 0; w < SL; ++w) {
    mt[w] = -finf;
    picked[w] = 64 * w + lane == pick;
  }
  for (int t = 1; t < kk; ++t) {
    const int p = pick;
    const float inv_p = s.inv32[p];
    const int tp = tri(p);
    // every slot reads (rows past the count read row c - 1 and are ignored),
    // so the reads of all slots go out together
    float g[SL];
#pragma unroll
    for (int w = 0; w < SL; ++w) {
      const int jj = min(64 * w + lane, c - 1);
      g[w] = s.gram[jj < p ? tp + jj : trij[w] + p];
    }
    uint32_t a = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < SL; ++w) {
      const int j = 64 * w + lane;
      const bool live = j < c && !picked[w];
      mt[w] = fmaxf(mt[w], (g[w] * invj[w]) * inv_p);
      a = min(a, live ? cand_key(mt[w], j) : 0xFFFFFFFFu);
    }
    const uint32_t k1 = wave_min_key(a);
    const float hi1 = key_hi(k1) + eps2;
    uint64_t inmask[SL];
    int inwin = 0;
#pragma unroll
    for (int w = 0; w < SL; ++w) {
      inmask[w] = __ballot(64 * w + lane < c && !picked[w] && mt[w] <= hi1);
      inwin += __builtin_popcountll(inmask[w]);
    }
    if (inwin > 1) {
      __builtin_amdgcn_wave_barrier();
      pick = fps_exact_argmin<DT, D, SL>(src, s, inmask, c, t, false);
    } else {
      pick = (int)(k1 & 0xFFu);
    }
#pragma unroll
    for (int w = 0; w < SL; ++w) picked[w] = picked[w] || (64 * w + lane == pick);
    if (lane == 0) s.picks[t] = pick;
  }
  __builtin_amdgcn_wave_barrier();
  if constexpr (kHold) fps_write_picks<DT, D, NT>(s, kk, fr, wb, lane);
  return kk;
}

// ---------------------------------------------------------------------------
// FPS of one head by NT cooperating waves
// ---------------------------------------------------------------------------
//
// Wave w owns the 32 rows of tile w as candidates.  Lane (n, h) holds half of
// row 32 w + n in matrix-core fragments (h = lane / 32), and, after the Gram
// step, the column G(., 32 w + n) for the rows i with (i % 8) / 4 == h:
// gc[16 t + r] = G(32 t + 8 (r / 4) + 4 h + r % 4, 32 w + n), the layout of
// the MFMA accumulator of tile pair (t, w).  A greedy round reads its pick's
// entry by a uniform register index (and the partner half by a lane swap),
// so no Gram matrix is kept in LDS.  Each round the waves publish
// their smallest and second-smallest candidate key in LDS; after one
// barrier every wave knows the best key k1 and the runner-up k2.  If k2's
// bucket starts above key_hi(k1) + window, k1's row is the binary64 argmin;
// otherwise the candidates within the window are decided in binary64 by
// wave 0 (a superset of the single-wave test, so never fewer binary64
// decisions).

struct FpsCoopLds {
  unsigned char* stage;  // [M][D] storage: picks staged for the buffer write-back
  float* inv32;          // [cap] fp32 1 / |x| (0 for rows past the count)
  int* map;              // [cap]
  int* picks;            // [cap]
  int* pos;              // [cap]
  uint32_t* pub;         // [2][NT][2]: smallest and second-smallest key per wave, by round parity
  uint32_t* mask;        // [NT]: window members of each wave's tile (bit n = row 32 w + n)
  int* flags;            // [NT]: per-wave unsafe-norm flag
  int* slot;             // [1]: pick of a binary64 decision
};

template <int DT, int D>
__host__ __device__ constexpr size_t fps_coop_stage_bytes(int M) {
  return ((size_t)M * D * Elem<DT>::kBytes + 15) & ~(size_t)15;
}

template <int DT, int D>
__host__ __device__ constexpr size_t fps_coop_lds_bytes(int NT, int M) {
  return fps_coop_stage_bytes<DT, D>(M) + (size_t)32 * NT * 16 + (size_t)NT * (16 + 4 + 4) + 16;
}

template <int DT, int D>
__device__ inline FpsCoopLds fps_coop_carve(unsigned char* smem, int NT, int M) {
  const int cap = 32 * NT;
  FpsCoopLds s;
  s.stage = smem;
  unsigned char* p = smem + fps_coop_stage_bytes<DT, D>(M);
  s.inv32 = reinterpret_cast<float*>(p);
  s.map = reinterpret_cast<int*>(p + (size_t)cap * 4);
  s.picks = reinterpret_cast<int*>(p + (size_t)cap * 8);
  s.pos = reinterpret_cast<int*>(p + (size_t)cap * 12);
  s.pub = reinterpret_cast<uint32_t*>(p + (size_t)cap * 16);
  s.mask = s.pub + 4 * NT;
  s.flags = reinterpret_cast<int*>(s.mask + NT);
  s.slot = s.flags + NT;
  return s;
}

// Lowest value of a key's bucket.
__device__ inline float key_lo(uint32_t k) {
  const uint32_t ord = k & 0xFFFFFF00u;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// One FPS decision of the block (see above).  `key` and `val` are this
// lane's candidate key (0xFFFFFFFF if none) and its fp32 objective; both
// lanes of a row hold the same.  Every thread must call it; the result is
// uniform.
template <int DT, int D, int NT>
__device__ __attribute__((always_inline)) int coop_decide(uint32_t key, float val, float win, int parity,
                                                          const FpsRows<DT, D>& src, const FpsCoopLds& s, int c,
                                                          int npicked, bool sum_mode) {
  constexpr int SL = (NT + 1) / 2;
  const int lane = fps_lane();
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const uint32_t k1w = wave_min_key(key);
  const uint32_t k2w = wave_min_key(key == k1w ? 0xFFFFFFFFu : key);
  uint32_t* pub = s.pub + 2 * NT * parity;
  if (lane == 0) {
    pub[2 * wv] = k1w;
    pub[2 * wv + 1] = k2w;
  }
  __syncthreads();
  uint32_t k1 = 0xFFFFFFFFu, k2 = 0xFFFFFFFFu;
#pragma unroll
  for (int w = 0; w < NT; ++w) {
    const uint32_t a = pub[2 * w], b = pub[2 * w + 1];
    if (a < k1) {
      k2 = min(k1, b);
      k1 = a;
    } else {
      k2 = min(k2, a);
    }
  }
  k1 = (uint32_t)__builtin_amdgcn_readfirstlane((int)k1);
  k2 = (uint32_t)__builtin_amdgcn_readfirstlane((int)k2);
  const float hi1 = key_hi(k1) + win;
  if (k2 == 0xFFFFFFFFu || key_lo(k2) > hi1) return (int)(k1 & 0xFFu);
  // binary64 decision over the candidates within the window (k1's own row
  // always among them, so the set is never empty)
  const uint64_t m = __ballot((lane >> 5) == 0 && key != 0xFFFFFFFFu && (val <= hi1 || key == k1));
  if (lane == 0) s.mask[wv] = (uint32_t)m;
  __syncthreads();
  if (wv == 0) {
    uint64_t inmask[SL];
#pragma unroll
    for (int q = 0; q < SL; ++q)
      inmask[q] = (uint64_t)s.mask[2 * q] | ((2 * q + 1 < NT) ? ((uint64_t)s.mask[2 * q + 1] << 32) : 0ull);
    // rare path: small load batches keep its registers below the rounds' own
    const int p = fps_exact_argmin<DT, D, SL, FpsCoopLds, 2>(src, s, inmask, c, npicked, sum_mode);
    if (lane == 0) *s.slot = p;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*s.slot);
}

// Rows of the picks written to wb + i d (pick i) from the fragments of their
// owner waves; no-op when wb is null.  Every thread of the block must call it.
template <int DT, int D, int NT>
__device__ __forceinline__ void coop_write_picks(const FpsCoopLds& s, int kk,
                                                 const typename FpsFrag<DT, D>::V (&fr)[FpsFrag<DT, D>::kSteps],
                                                 typename Elem<DT>::T* wb, int j, int h, bool inrow) {
  using FR = FpsFrag<DT, D>;
  if (wb == nullptr) return;
  for (int r = threadIdx.x; r < 32 * NT; r += 64 * NT) s.pos[r] = -1;
  __syncthreads();
  for (int i = threadIdx.x; i < kk; i += 64 * NT) s.pos[s.picks[i]] = i;
  __syncthreads();
  const int i = s.pos[j];
  if (inrow && i >= 0) {
#pragma unroll
    for (int ks = 0; ks < FR::kSteps; ++ks) FR::store(wb + (size_t)i * D, ks, h, fr[ks]);
  }
}

// Writes the FPS picks of rows [0, c) (c <= 32 NT) to s.picks, min(k, c) of
// them, and returns the count.  When `wb` is given, also writes pick i's row
// to wb + i d from the owner waves' fragments.  Every thread of the block
// (64 NT) must call it.
template <int DT, int D, int NT>
__device__ __attribute__((always_inline)) int fps_coop(const FpsRows<DT, D>& src, const FpsCoopLds& s, int c, int k,
                                                       typename Elem<DT>::T* wb = nullptr) {
  using FR = FpsFrag<DT, D>;
  using V = typename FR::V;
  using T = typename Elem<DT>::T;
  constexpr int KS = FR::kSteps;
  constexpr int SL = (NT + 1) / 2;
  constexpr float kEps = 4.0f * (D + 8) * kFpsU;
  const int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  int lane = fps_lane();
  __asm__ volatile("" : "+v"(lane));
  const int wv = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int n = lane & 31, h = lane >> 5;
  const int j = 32 * wv + n;  // this lane's candidate row
  const bool inrow = j < c;
  const float finf = __builtin_huge_valf();

  // 1. fragments of this wave's rows (rows past the count read row c - 1 and are zeroed)
  V fr[KS];
  {
    const T* rp = src.row(min(j, c - 1));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V v = FR::load(rp, ks, h);
      fr[ks] = inrow ? v : FR::zero();
    }
  }

  // 2. fp32 inverse norm of row j (both lanes of the row hold it)
  float inv = 0.0f;
  int unsafe = 0;
  {
    float ss = 0.0f;
    uint32_t nz = 0;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ss = FR::sumsq(fr[ks], ss);
      nz |= FR::nonzero(fr[ks]);
    }
    ss += __shfl_xor(ss, 32, 64);
    nz |= (uint32_t)__shfl_xor((int)nz, 32, 64);
    if (inrow) {
      if (ss > 0.0f) {
        if (!(ss >= 1e-30f && ss <= 1e36f)) unsafe = 1;
        inv = (float)(1.0 / sqrt((double)ss));
      } else {
        if (nz) unsafe = 1;  // nonzero row whose fp32 squares underflow
        inv = 1e12f;         // zero row: norm clamped at 1e-12, every cosine 0
      }
    }
    if (h == 0) s.inv32[j] = inv;
    const bool wunsafe = __ballot(unsafe) != 0;
    if (lane == 0) s.flags[wv] = wunsafe ? 1 : 0;
  }
  __syncthreads();
  int any_unsafe = 0;
#pragma unroll
  for (int w = 0; w < NT; ++w) any_unsafe |= s.flags[w];

  if (any_unsafe) {  // binary64 rounds over every candidate, by wave 0
    if (wv == 0) {
      uint64_t avail[SL];
#pragma unroll
      for (int q = 0; q < SL; ++q) {
        const int cnt = c - 64 * q;
        avail[q] = cnt >= 64 ? ~0ull : (cnt > 0 ? ((1ull << cnt) - 1) : 0ull);
      }
      for (int t = 0; t < kk; ++t) {
        const int pick = fps_exact_argmin<DT, D, SL, FpsCoopLds, 2>(src, s, avail, c, t, t == 0);
#pragma unroll
        for (int q = 0; q < SL; ++q)
          if ((pick >> 6) == q) avail[q] &= ~(1ull << (pick & 63));
        if (lane == 0) s.picks[t] = pick;
        __builtin_amdgcn_wave_barrier();
      }
    }
    __syncthreads();
    coop_write_picks<DT, D, NT>(s, kk, fr, wb, j, h, inrow);
    return kk;
  }

  // 3. Gram columns of this wave's candidates, one 32-row tile at a time
  // (straight-line MFMA chains); one 16-float vector per tile, so that a
  // uniform element index stays a register move
  fps_floatx16 gc[NT];
#pragma unroll
  for (int tr = 0; tr < NT; ++tr) {
    const int ri = 32 * tr + n;
    const T* rp = src.row(min(ri, c - 1));
    V a[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const V v = FR::load(rp, ks, h);
      a[ks] = ri < c ? v : FR::zero();
    }
    fps_floatx16 acc = fps_floatx16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = FR::mma(a[ks], fr[ks], acc);
    gc[tr] = acc;
    // one tile's rows in registers at a time (other waves hide the latency)
    __builtin_amdgcn_sched_barrier(0);
  }

  // 4. start: lowest mean cosine, from this column's sum of G_ij / |x_i|
  int pick;
  {
    float cs = 0.0f;
#pragma unroll
    for (int tr = 0; tr < NT; ++tr) {
      const float4* ivp = reinterpret_cast<const float4*>(s.inv32 + 32 * tr + 4 * h);
      const float4 iv[4] = {ivp[0], ivp[2], ivp[4], ivp[6]};
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float4 q = iv[r >> 2];
        const float w = (r & 3) == 0 ? q.x : (r & 3) == 1 ? q.y : (r & 3) == 2 ? q.z : q.w;
        cs = fmaf(gc[tr][r], w, cs);
      }
    }
    cs += __shfl_xor(cs, 32, 64);
    const float mu = inrow ? (cs * inv) / (float)c : finf;
    const float eps_mu = kEps + 4.0f * (float)(c + 8) * kFpsU;
    pick = coop_decide<DT, D, NT>(inrow ? cand_key(mu, j) : 0xFFFFFFFFu, mu, 2.0f * eps_mu, 0, src, s, c, 0, true);
  }
  if (threadIdx.x == 0) s.picks[0] = pick;

  // 5. greedy rounds on fp32 cosines
  const float eps2 = 2.0f * kEps;
  float mt = -finf;
  bool picked = j == pick;
  for (int t = 1; t < kk; ++t) {
    const int p = pick;
    const float inv_p = s.inv32[p];
    const int pr = 4 * ((p & 31) >> 3) + (p & 3);  // uniform element index within tile p / 32
    float vo = 0.0f;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const float x = gc[q][pr];
      vo = (q == (p >> 5)) ? x : vo;
    }
    const float vp = __shfl_xor(vo, 32, 64);
    const float g = (h == ((p >> 2) & 1)) ? vo : vp;
    mt = fmaxf(mt, (g * inv) * inv_p);
    const bool live = inrow && !picked;
    pick = coop_decide<DT, D, NT>(live ? cand_key(mt, j) : 0xFFFFFFFFu, mt, eps2, t & 1, src, s, c, t, false);
    picked = picked || (j == pick);
    if (threadIdx.x == 0) s.picks[t] = pick;
  }
  __syncthreads();
  coop_write_picks<DT, D, NT>(s, kk, fr, wb, j, h, inrow);
  return kk;
}


// Copies n 16-byte units, unit u from src_at(u) to dst_at(u, v), over the
// block's NTH threads with eight loads per thread in flight (clamped in
// bounds) ahead of their stores.
template <int NTH, typename SrcF, typename DstF>
__device__ inline void copy_units_n(int n, SrcF src_at, DstF dst_at) {
  const int l = threadIdx.x;
  for (int u0 = 0; u0 < n; u0 += 8 * NTH) {
    const int m = n - 1;
    const uint4 v0 = src_at(min(u0 + l, m));
    const uint4 v1 = src_at(min(u0 + NTH + l, m));
    const uint4 v2 = src_at(min(u0 + 2 * NTH + l, m));
    const uint4 v3 = src_at(min(u0 + 3 * NTH + l, m));
    const uint4 v4 = src_at(min(u0 + 4 * NTH + l, m));
    const uint4 v5 = src_at(min(u0 + 5 * NTH + l, m));
    const uint4 v6 = src_at(min(u0 + 6 * NTH + l, m));
    const uint4 v7 = src_at(min(u0 + 7 * NTH + l, m));
    if (u0 + l < n) dst_at(u0 + l, v0);
    if (u0 + NTH + l < n) dst_at(u0 + NTH + l, v1);
    if (u0 + 2 * NTH + l < n) dst_at(u0 + 2 * NTH + l, v2);
    if (u0 + 3 * NTH + l < n) dst_at(u0 + 3 * NTH + l, v3);
    if (u0 + 4 * NTH + l < n) dst_at(u0 + 4 * NTH + l, v4);
    if (u0 + 5 * NTH + l < n) dst_at(u0 + 5 * NTH + l, v5);
    if (u0 + 6 * NTH + l < n) dst_at(u0 + 6 * NTH + l, v6);
    if (u0 + 7 * NTH + l < n) dst_at(u0 + 7 * NTH + l, v7);
  }
}


// Copies n 16-byte units, unit u from src_at(u) to dst_at(u, v), with kB
// loads per lane in flight (clamped in bounds) ahead of their stores.
template <int kB = 8, typename SrcF, typename DstF>
__device__ inline void copy_units(int n, SrcF src_at, DstF dst_at) {
  const int l = fps_lane();
  for (int u0 = 0; u0 < n; u0 += 64 * kB) {
    const int m = n - 1;
    uint4 v[kB];
#pragma unroll
    for (int b = 0; b < kB; ++b) v[b] = src_at(min(u0 + 64 * b + l, m));
#pragma unroll
    for (int b = 0; b < kB; ++b)
      if (u0 + 64 * b + l < n) dst_at(u0 + 64 * b + l, v[b]);
  }
}

// ---------------------------------------------------------------------------
// Ingest
// ---------------------------------------------------------------------------

template <int DT, int D, int NT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void fps_update_kernel(
    const typename Elem<DT>::T* __restrict__ q_new, int T, typename Elem<DT>::T* __restrict__ qbuf,
    int32_t* __restrict__ qcount, int C, int M, int32_t* __restrict__ ws_words) {
  using ET = typename Elem<DT>::T;
  constexpr int kRowBytes = D * Elem<DT>::kBytes;
  constexpr int kU = kRowBytes / 16;
  constexpr int cap = 32 * NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x;
  const int lane = fps_lane();
  ET* buf = qbuf + (size_t)head * C * D;
  const ET* qn = q_new + (size_t)head * T * D;
  const int c0 = qcount[head];
  if (c0 < 0 || c0 >= C) {
    if (lane == 0) set_status(ws_words, BKV_DEV_BAD_COUNT);
    return;
  }
  if (c0 + T < C) {  // no shrink in this call: plain append
    copy16(buf + (size_t)c0 * D, qn, T * kRowBytes, lane, 64);
    if (lane == 0) qcount[head] = c0 + T;
    return;
  }
  FpsLds s = fps_carve<DT, D>(smem, cap, M);
  const FpsRows<DT, D> src{buf, qn, s.map, C};
  for (int r = lane; r < c0; r += 64) s.map[r] = r;
  int c = c0, t = 0, nlast = 0;
  bool written = false;
  while (t < T) {
    const int take = (T - t) < (C - c) ? (T - t) : (C - c);
    for (int u = lane; u < take; u += 64) s.map[c + u] = C + t + u;
    c += take;
    t += take;
    __builtin_amdgcn_wave_barrier();
    if (c == C) {
      // the last shrink of the call (no refill from the remaining arrivals)
      // writes its picks to the buffer from registers; an earlier one turns
      // the buffer into its picks through the row map
      const bool direct = fps_holds<DT, D, NT>() && M + (T - t) < C;
      const int np = fps_wave<DT, D, NT>(src, s, C, M, direct ? buf : nullptr);
      if (direct) {
        written = true;
      } else {
        constexpr int kQ = (cap + 63) / 64;
        int nm[kQ];
#pragma unroll
        for (int q = 0; q < kQ; ++q) nm[q] = s.map[s.picks[min(lane + 64 * q, np - 1)]];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int q = 0; q < kQ; ++q) {
          const int i = lane + 64 * q;
          if (i < np) s.map[i] = nm[q];
        }
        __builtin_amdgcn_wave_barrier();
      }
      c = np;
      nlast = np;
    }
  }
  uint4* bufu = reinterpret_cast<uint4*>(buf);
  if (!written) {
    // the retained picks may be rows of the entry buffer, so they are staged
    // in LDS before any row of the buffer is overwritten
    uint4* stage = reinterpret_cast<uint4*>(s.stage);
    copy_units(nlast * kU, [&](int u) { return reinterpret_cast<const uint4*>(src.row(u / kU))[u % kU]; },
               [&](int u, uint4 v) { stage[u] = v; });
    __builtin_amdgcn_wave_barrier();
    copy_units(nlast * kU, [&](int u) { return stage[u]; }, [&](int u, uint4 v) { bufu[u] = v; });
  }
  // the rows after the picks are the last arrivals of the call, contiguous
  // in q_new (the fragments are dead by now, so more loads fit in flight)
  if (c > nlast) {
    const uint4* tail = reinterpret_cast<const uint4*>(src.row(nlast));
    uint4* dst = bufu + (size_t)nlast * kU;
    copy_units<16>((c - nlast) * kU, [&](int u) { return tail[u]; }, [&](int u, uint4 v) { dst[u] = v; });
  }
  if (lane == 0) qcount[head] = c;
}

// ---------------------------------------------------------------------------
// RoPE tables: (cos, sin) per slot for the R recent positions and pos_now
// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Beacon selection: FPS over the live buffer of each query head
// ---------------------------------------------------------------------------

// Waves per SIMD a beacon-pick wave's registers are budgeted for: one tile
// of rows leaves room for four, more tiles for two.
template <int NT>
constexpr int picks_waves_per_simd() {
  return NT == 1 ? 4 : 2;
}


// One wavefront per query head whose live count c lies in (cmin, cmax], a
// range within one tile count NT (the launch for one tile takes c = 0 and the
// heads whose count is out of range too); the other heads are left to the
// launches for their tile count, so that each kernel holds only one tile
// count's fragments and Gram triangle.
// Writes beacons[head][0] = the pick count min(nb, count), beacons[head][1 +
// b] = buffer row of pick b, in pick order, and a copy of the picked rows to
// rows[head][b] (so that scoring does not read the buffer, which the next
// ingest may already be changing).  The score kernel rotates them.
template <int DT, int D, int NT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, picks_waves_per_simd<NT>()))) void
beacon_pick_kernel(const typename Elem<DT>::T* __restrict__ qbuf, const int32_t* __restrict__ qcount, int C, int nb,
                   int32_t* __restrict__ beacons, typename Elem<DT>::T* __restrict__ rows,
                   int32_t* __restrict__ ws_words, int cmin, int cmax) {
  constexpr int cap = 32 * NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x;
  const int lane = fps_lane();
  int c = qcount[head];
  if (c < 0 || c >= C) {
    if (lane == 0) set_status(ws_words, BKV_DEV_BAD_COUNT);
    c = 0;
  }
  if (c <= cmin || c > cmax) return;  // another tile count's launch takes the head
  const int want = nb < c ? nb : c;
  FpsLds s = fps_carve<DT, D>(smem, cap, 0);
  const FpsRows<DT, D> src{qbuf + (size_t)head * C * D, nullptr, s.map, C};
  int kk = 0;
  if (want > 0) {
    for (int r = lane; r < c; r += 64) s.map[r] = r;
    __builtin_amdgcn_wave_barrier();
    kk = fps_wave<DT, D, NT>(src, s, c, want);
  }
  int32_t* out = beacons + (size_t)head * (nb + 1);
  for (int b = lane; b < kk; b += 64) out[1 + b] = s.picks[b];
  if (lane == 0) out[0] = kk;
  // the picked rows, 16 bytes per lane and load
  constexpr int kU = D * Elem<DT>::kBytes / 16;
  uint4* dst = reinterpret_cast<uint4*>(rows + (size_t)head * nb * D);
  for (int u = lane; u < kk * kU; u += 64) {
    const int b = u / kU, q = u - b * kU;
    dst[u] = reinterpret_cast<const uint4*>(src.row(s.picks[b]))[q];
  }
}

// One workgroup of NT waves per query head (NT = 32-row tiles of C).
template <int DT, int D, int NT>
__global__ __launch_bounds__(64 * NT) void fps_update_coop_kernel(const typename Elem<DT>::T* __restrict__ q_new, int T,
                                                             typename Elem<DT>::T* __restrict__ qbuf,
                                                             int32_t* __restrict__ qcount, int C, int M,
                                                             int32_t* __restrict__ ws_words) {
  constexpr int NTH = 64 * NT;
  constexpr int kRowBytes = D * Elem<DT>::kBytes;
  constexpr int kU = kRowBytes / 16;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  using ET = typename Elem<DT>::T;
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  ET* buf = qbuf + (size_t)head * C * D;
  const ET* qn = q_new + (size_t)head * T * D;
  const int c0 = qcount[head];
  if (c0 < 0 || c0 >= C) {
    if (tid == 0) set_status(ws_words, BKV_DEV_BAD_COUNT);
    return;
  }
  if (c0 + T < C) {  // no shrink in this call: plain append
    copy16(buf + (size_t)c0 * D, qn, T * kRowBytes, tid, NTH);
    if (tid == 0) qcount[head] = c0 + T;
    return;
  }
  FpsCoopLds s = fps_coop_carve<DT, D>(smem, NT, M);
  const FpsRows<DT, D> src{buf, qn, s.map, C};
  for (int r = tid; r < c0; r += NTH) s.map[r] = r;
  int c = c0, t = 0, nlast = 0;
  while (t < T) {
    const int take = (T - t) < (C - c) ? (T - t) : (C - c);
    for (int u = tid; u < take; u += NTH) s.map[c + u] = C + t + u;
    c += take;
    t += take;
    __syncthreads();
    if (c == C) {
      // the buffer becomes its picks through the row map
      const int np = fps_coop<DT, D, NT>(src, s, C, M);
      const int nm = tid < np ? s.map[s.picks[tid]] : 0;  // np <= M < C <= NTH / 2
      __syncthreads();
      if (tid < np) s.map[tid] = nm;
      __syncthreads();
      c = np;
      nlast = np;
    }
  }
  uint4* bufu = reinterpret_cast<uint4*>(buf);
  {
    // the retained picks may be rows of the entry buffer, so they are staged
    // in LDS before any row of the buffer is overwritten
    uint4* stage = reinterpret_cast<uint4*>(s.stage);
    copy_units_n<NTH>(nlast * kU, [&](int u) { return reinterpret_cast<const uint4*>(src.row(u / kU))[u % kU]; },
                    [&](int u, uint4 v) { stage[u] = v; });
    __syncthreads();
    copy_units_n<NTH>(nlast * kU, [&](int u) { return stage[u]; }, [&](int u, uint4 v) { bufu[u] = v; });
  }
  // the rows after the picks are the last arrivals of the call, contiguous in q_new
  if (c > nlast) {
    const uint4* tail = reinterpret_cast<const uint4*>(src.row(nlast));
    uint4* dst = bufu + (size_t)nlast * kU;
    copy_units_n<NTH>((c - nlast) * kU, [&](int u) { return tail[u]; }, [&](int u, uint4 v) { dst[u] = v; });
  }
  if (tid == 0) qcount[head] = c;
}

// One workgroup of NT waves per query head (capacities above 128 rows).  Writes beacons[head][0] = the pick count
// min(nb, count), beacons[head][1 + b] = buffer row of pick b, in pick
// order, and a copy of the picked rows to rows[head][b] (so that scoring
// does not read the buffer, which the next ingest may already be changing).
// The score kernel rotates them.
template <int DT, int D, int NT>
__global__ __launch_bounds__(64 * NT) void beacon_pick_coop_kernel(const typename Elem<DT>::T* __restrict__ qbuf,
                                                              const int32_t* __restrict__ qcount, int C, int nb,
                                                              int32_t* __restrict__ beacons,
                                                              typename Elem<DT>::T* __restrict__ rows,
                                                              int32_t* __restrict__ ws_words, int cmin) {
  constexpr int NTH = 64 * NT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  int c = qcount[head];
  if (c < 0 || c >= C) {
    if (tid == 0) set_status(ws_words, BKV_DEV_BAD_COUNT);
    c = 0;
  }
  if (c <= cmin) return;  // few enough live rows for the single-wave kernel, which takes the head
  const int want = nb < c ? nb : c;
  FpsCoopLds s = fps_coop_carve<DT, D>(smem, NT, 0);
  const FpsRows<DT, D> src{qbuf + (size_t)head * C * D, nullptr, s.map, C};
  int kk = 0;
  if (want > 0) {
    for (int r = tid; r < c; r += NTH) s.map[r] = r;
    __syncthreads();
    kk = fps_coop<DT, D, NT>(src, s, c, want);
  }
  int32_t* out = beacons + (size_t)head * (nb + 1);
  for (int b = tid; b < kk; b += NTH) out[1 + b] = s.picks[b];
  if (tid == 0) out[0] = kk;
  // the picked rows, 16 bytes per thread and load
  constexpr int kU = D * Elem<DT>::kBytes / 16;
  uint4* dst = reinterpret_cast<uint4*>(rows + (size_t)head * nb * D);
  for (int u = tid; u < kk * kU; u += NTH) {
    const int b = u / kU, q = u - b * kU;
    dst[u] = reinterpret_cast<const uint4*>(src.row(s.picks[b]))[q];
  }
}

// Beacons given by the caller instead of chosen by FPS (the policy variants
// the pages compare against: the earliest queries of a head, or rows drawn at
// random from its buffer).  Head h takes rows idx[h][0, cnt) of its source
// src[h][S][row], where cnt is the length of the leading run of entries in
// [0, S); a negative entry ends the list, an entry >= S ends it too and sets
// BKV_DEV_BAD_INDEX.  Writes the same workspace regions as beacon_pick_kernel.
__global__ __launch_bounds__(64) void beacon_rows_kernel(const unsigned char* __restrict__ src, int S,
                                                         const int32_t* __restrict__ idx, int nb, int row_bytes,
                                                         int32_t* __restrict__ beacons,
                                                         unsigned char* __restrict__ rows,
                                                         int32_t* __restrict__ ws_words) {
  const size_t head = blockIdx.x;
  const int lane = threadIdx.x;
  const int32_t* ih = idx + head * nb;
  int stop = nb;  // first entry outside [0, S)
  for (int b = lane; b < nb; b += 64)
    if (ih[b] < 0 || ih[b] >= S) stop = min(stop, b);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) stop = min(stop, __shfl_xor(stop, off, 64));
  if (lane == 0 && stop < nb && ih[stop] >= S) set_status(ws_words, BKV_DEV_BAD_INDEX);
  int32_t* out = beacons + head * (nb + 1);
  for (int b = lane; b < stop; b += 64) out[1 + b] = ih[b];
  if (lane == 0) out[0] = stop;
  const int ku = row_bytes / 16;
  const unsigned char* sh = src + head * (size_t)S * row_bytes;
  uint4* dst = reinterpret_cast<uint4*>(rows + head * (size_t)nb * row_bytes);
  for (int u = lane; u < stop * ku; u += 64) {
    const int b = u / ku, q = u - b * ku;
    dst[u] = reinterpret_cast<const uint4*>(sh + (size_t)ih[b] * row_bytes)[q];
  }
}

hipError_t launch_beacon_rows(const void* src, int S, const int32_t* idx, int nb, int row_bytes, int heads,
                              int32_t* beacons, void* rows, int32_t* ws_words, hipStream_t st) {
  hipLaunchKernelGGL(beacon_rows_kernel, dim3(heads), dim3(64), 0, st, (const unsigned char*)src, S, idx, nb,
                     row_bytes, beacons, (unsigned char*)rows, ws_words);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launchers (tile capacity from the buffer capacity)
// ---------------------------------------------------------------------------

template <int DT, int D, int NT>
static hipError_t launch_fps_update_nt(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M,
                                       int heads, int32_t* ws_words, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const size_t smem = fps_lds_bytes<DT, D>(32 * NT, M);
  auto kern = fps_update_kernel<DT, D, NT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(64), smem, st, (const ET*)q_new, T, (ET*)qbuf, qcount, C, M,
                     ws_words);
  return hipGetLastError();
}

// Capacities above 128 rows: one workgroup of eight waves per head (the
// single-wave kernel's 130 KB Gram triangle would leave one wave per CU).
template <int DT, int D>
static hipError_t launch_fps_update_coop(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M,
                                         int heads, int32_t* ws_words, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  constexpr int NT = 8;
  const size_t smem = fps_coop_lds_bytes<DT, D>(NT, M);
  auto kern = fps_update_coop_kernel<DT, D, NT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(64 * NT), smem, st, (const ET*)q_new, T, (ET*)qbuf, qcount, C, M,
                     ws_words);
  return hipGetLastError();
}

// one instantiation per 32-row tile count of the capacity up to 4 tiles; the
// cooperative kernel above that
template <int DT, int D>
hipError_t launch_fps_update(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M, int heads,
                             int32_t* ws_words, hipStream_t st) {
  switch ((C + 31) / 32) {
    case 1: return launch_fps_update_nt<DT, D, 1>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
    case 2: return launch_fps_update_nt<DT, D, 2>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
    case 3: return launch_fps_update_nt<DT, D, 3>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
    case 4: return launch_fps_update_nt<DT, D, 4>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
    default: return launch_fps_update_coop<DT, D>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
  }
}

template <int DT, int D, int NT>
static hipError_t launch_picks_nt(const void* qbuf, const int32_t* qcount, int C, int nb, int heads,
                                  int32_t* beacons, void* rows, int32_t* ws_words, hipStream_t st) {
  static_assert(NT >= 1 && NT <= 4, "one to four tiles of 32 rows");
  using ET = typename Elem<DT>::T;
  const size_t smem = fps_lds_bytes<DT, D>(32 * NT, 0);
  auto kern = beacon_pick_kernel<DT, D, NT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  // live counts (32 (NT - 1), 32 NT]; the one-tile launch also takes 0
  hipLaunchKernelGGL(kern, dim3(heads), dim3(64), smem, st, (const ET*)qbuf, qcount, C, nb, beacons, (ET*)rows,
                     ws_words, NT == 1 ? -1 : 32 * (NT - 1), 32 * NT);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_picks_coop(const void* qbuf, const int32_t* qcount, int C, int nb, int heads,
                                    int32_t* beacons, void* rows, int32_t* ws_words, int cmin, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  constexpr int NT = 8;
  const size_t smem = fps_coop_lds_bytes<DT, D>(NT, 0);
  auto kern = beacon_pick_coop_kernel<DT, D, NT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(64 * NT), smem, st, (const ET*)qbuf, qcount, C, nb, beacons,
                     (ET*)rows, ws_words, cmin);
  return hipGetLastError();
}

// One launch per 32-row tile count of the live rows up to four tiles (each
// launch skips the heads of the others), the cooperative kernel for heads
// with more than 128 live rows.
template <int DT, int D>
hipError_t launch_beacon_picks(const void* qbuf, const int32_t* qcount, int C, int nb, int heads, int32_t* beacons,
                               void* rows, int32_t* ws_words, hipStream_t st) {
  hipError_t e = launch_picks_nt<DT, D, 1>(qbuf, qcount, C, nb, heads, beacons, rows, ws_words, st);
  if (e == hipSuccess && C > 32) e = launch_picks_nt<DT, D, 2>(qbuf, qcount, C, nb, heads, beacons, rows, ws_words, st);
  if (e == hipSuccess && C > 64) e = launch_picks_nt<DT, D, 3>(qbuf, qcount, C, nb, heads, beacons, rows, ws_words, st);
  if (e == hipSuccess && C > 96) e = launch_picks_nt<DT, D, 4>(qbuf, qcount, C, nb, heads, beacons, rows, ws_words, st);
  if (e == hipSuccess && C > 128) e = launch_picks_coop<DT, D>(qbuf, qcount, C, nb, heads, beacons, rows, ws_words, 128, st);
  return e;
}

template hipError_t launch_fps_update<BKV_F32, 64>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                   hipStream_t);
template hipError_t launch_fps_update<BKV_F32, 128>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                    hipStream_t);
template hipError_t launch_fps_update<BKV_BF16, 64>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                    hipStream_t);
template hipError_t launch_fps_update<BKV_BF16, 128>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                     hipStream_t);
#define BKV_INST_PICKS(DT, D)                                                                                  \
  template hipError_t launch_beacon_picks<DT, D>(const void*, const int32_t*, int, int, int, int32_t*, void*,      \
                                                 int32_t*, hipStream_t);
BKV_INST_PICKS(BKV_F32, 64)
BKV_INST_PICKS(BKV_F32, 128)
BKV_INST_PICKS(BKV_BF16, 64)
BKV_INST_PICKS(BKV_BF16, 128)

}  // namespace bkv

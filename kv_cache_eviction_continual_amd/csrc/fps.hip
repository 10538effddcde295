// fps.hip -- Continual farthest point sampling on gfx950.
//
// Two kernels share one FPS routine:
//   fps_update_kernel  ingest of new pre-RoPE queries into the bounded
//                      per-query-head buffer, shrinking it by FPS whenever it
//                      fills (wzjinhao.cn news article 56682 on BeaconKV,
//                      section 怎么挑出这几个信标: bounded buffer per head,
//                      FPS compression back to a smaller size when full);
//   obs_build_kernel   beacon selection by FPS over the live buffer, then
//                      RoPE of the beacons (to the current decode position)
//                      and of the recent queries (to their own positions)
//                      into the observation rows the score kernel consumes
//                      (same article, section 信标查询怎么用).
//
// FPS on cosine similarity: start at the row with the lowest mean cosine to
// all rows; then repeatedly add the row with the lowest maximum cosine to the
// picked set; ties go to the lower row.
//
// The decisions are those of binary64 evaluation:
//   * the start (mean cosines) is evaluated in binary64;
//   * the greedy rounds run on the Gram matrix X X^T from the matrix cores
//     (bf16 or fp32 products are exact, sums are fp32), which bounds the
//     error of every fp32 cosine by eps = 4 (d + 8) 2^-24 (fp32 dot-product
//     error bound gamma_d plus the normalisation roundings, doubled).  When
//     the best candidate is not ahead of the runner-up by more than 2 eps,
//     the maximum cosines of every candidate inside that window are
//     recomputed from the rows in binary64 and decide the pick;
//   * rows whose norms leave [1e-15, 1e18] (where fp32 Gram entries could
//     underflow or overflow) send the whole call to a plain binary64 path.
//
// One workgroup of 64 * NW threads per query head handles up to 32 * NW
// rows; thread i owns candidate row i.  The live buffer sits in LDS in its
// storage type (rows padded by 16 bytes); wave w keeps Gram rows
// [32 w, 32 w + 32) in its MFMA accumulators, and each pick publishes one
// Gram row through LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 fps_bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float fps_floatx16;

template <int DT, int D, int NW>
struct Fps {
  using E = Elem<DT>;
  using ET = typename E::T;
  static constexpr int NT = 64 * NW;
  static constexpr int kMaxRows = 32 * NW;
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kRowStride = kRowBytes + 16;
  static constexpr int kU = kRowBytes / 16;   // 16-byte units per row
  static constexpr int kPer16 = 16 / E::kBytes;
  static constexpr int kP = D / 32;           // lanes per exact dot product (32 dims each)
  static constexpr int kGroups = NT / kP;     // exact dot products per sweep
  static constexpr float kU32 = 5.9604644775390625e-8f;  // 2^-24
  static constexpr float kEps = 4.0f * (D + 8) * kU32;   // bound on |fp32 cosine - cosine|
};

struct FpsSmem {
  unsigned char* rows;  // row r at rows + r * kRowStride
  double* inv64;        // [kMaxRows] 1 / max(|x|, 1e-12), binary64
  float* inv32;         // [kMaxRows] the same, binary32
  float* colx;          // [NW][32] wave-private Gram column
  double* dslot;        // [2][NW] exact argmin values
  int* islot;           // [2][2 NW] argmin indices / candidate-key pairs
  int* picks;           // [kMaxRows]
  int* ulist;           // [kMaxRows] candidates inside an uncertain window
  double* uacc;         // [kMaxRows] their binary64 objectives
  double* pairv;        // [kGroups]
  int* pairu;           // [kGroups]
  int* misc;            // [16] block-scan scratch
};

template <int DT, int D, int NW>
__host__ __device__ constexpr size_t fps_smem_bytes(int nrows) {
  using F = Fps<DT, D, NW>;
  return (((size_t)nrows * F::kRowStride + 15) & ~(size_t)15) + F::kMaxRows * (8 + 4 + 4 + 4 + 8) +
         NW * 32 * 4 + 2 * NW * (8 + 4 + 4 + 8) + F::kGroups * (8 + 4) + 64 + 128;
}

template <int DT, int D, int NW>
__device__ inline FpsSmem fps_carve(unsigned char* smem, int nrows) {
  using F = Fps<DT, D, NW>;
  FpsSmem s;
  size_t off = ((size_t)nrows * F::kRowStride + 15) & ~(size_t)15;
  s.rows = smem;
  auto take = [&](size_t bytes) {
    unsigned char* p = smem + off;
    off += (bytes + 7) & ~(size_t)7;
    return p;
  };
  s.inv64 = reinterpret_cast<double*>(take(F::kMaxRows * 8));
  s.uacc = reinterpret_cast<double*>(take(F::kMaxRows * 8));
  s.dslot = reinterpret_cast<double*>(take(2 * NW * 8));
  s.pairv = reinterpret_cast<double*>(take(F::kGroups * 8));
  s.inv32 = reinterpret_cast<float*>(take(F::kMaxRows * 4));
  s.colx = reinterpret_cast<float*>(take(NW * 32 * 4));
  s.islot = reinterpret_cast<int*>(take(2 * 2 * NW * 4));
  s.picks = reinterpret_cast<int*>(take(F::kMaxRows * 4));
  s.ulist = reinterpret_cast<int*>(take(F::kMaxRows * 4));
  s.pairu = reinterpret_cast<int*>(take(F::kGroups * 4));
  s.misc = reinterpret_cast<int*>(take(64));
  return s;
}

template <int DT, int D, int NW>
__device__ inline const typename Elem<DT>::T* fps_row(const FpsSmem& s, int r) {
  return reinterpret_cast<const typename Elem<DT>::T*>(s.rows + (size_t)r * Fps<DT, D, NW>::kRowStride);
}

// binary64 dot product of dims [32 q, 32 q + 32) of rows a and b
template <int DT, int D, int NW>
__device__ inline double dot_slice64(const FpsSmem& s, int a, int b, int q) {
  using F = Fps<DT, D, NW>;
  using E = Elem<DT>;
  const uint4* xa = reinterpret_cast<const uint4*>(fps_row<DT, D, NW>(s, a) + 32 * q);
  const uint4* xb = reinterpret_cast<const uint4*>(fps_row<DT, D, NW>(s, b) + 32 * q);
  double acc = 0.0;
#pragma unroll 1
  for (int u = 0; u < 32 / F::kPer16; ++u) {
    const uint4 wa = xa[u], wb = xb[u];
    const typename E::T* ea = reinterpret_cast<const typename E::T*>(&wa);
    const typename E::T* eb = reinterpret_cast<const typename E::T*>(&wb);
#pragma unroll
    for (int k = 0; k < F::kPer16; ++k) acc = fma(E::to_f64(ea[k]), E::to_f64(eb[k]), acc);
  }
  return acc;
}

template <int P>
__device__ inline double sum_lanes(double v) {
#pragma unroll
  for (int off = 1; off < P; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Rotate a value within each 16-lane row of the wave (row_ror DPP).
template <int N>
__device__ inline float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}

// Sum over the 32 lanes of each half wave (every lane of the half gets a sum).
__device__ inline float half_wave_sum(float v) {
  v += row_ror<8>(v);
  v += row_ror<4>(v);
  v += row_ror<2>(v);
  v += row_ror<1>(v);
  return v + __shfl_xor(v, 16, 64);
}

// Block-wide argmin of (value, index); every thread gets the winning index.
template <int NW>
__device__ inline int block_argmin64(double v, int i, const FpsSmem& s, int& parity) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double ov = __shfl_xor(v, off, 64);
    const int oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s.dslot[parity * NW + wave] = v;
    s.islot[parity * NW + wave] = i;
  }
  __syncthreads();
  double bv = s.dslot[parity * NW];
  int bi = s.islot[parity * NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    const double ov = s.dslot[parity * NW + w];
    const int oi = s.islot[parity * NW + w];
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  parity ^= 1;
  return bi;
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
// Lowest value of a key's bucket, and the lowest value of the next bucket.
__device__ inline float key_lo(uint32_t k) {
  const uint32_t ord = k & 0xFFFFFF00u;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ inline float key_hi(uint32_t k) {
  const uint32_t ord = (k | 0xFFu) + 1u;
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

template <int N>
__device__ inline uint32_t row_ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x120 + N, 0xF, 0xF, false);
}

// Merge two (smallest, second smallest) key pairs of disjoint sets.
__device__ inline void merge2(uint32_t& a1, uint32_t& a2, uint32_t b1, uint32_t b2) {
  const uint32_t lo = a1 < b1 ? a1 : b1;
  const uint32_t hi = a1 < b1 ? b1 : a1;
  const uint32_t m2 = a2 < b2 ? a2 : b2;
  a1 = lo;
  a2 = hi < m2 ? hi : m2;
}

// Block-wide two smallest keys; candidates sit in lanes 0..31 of each wave
// (other lanes pass 0xFFFFFFFF).  Rows of 16 lanes reduce by DPP rotation,
// the two rows of the half wave through scalar lane reads, the waves through
// one LDS exchange.  Every thread returns the same pair.
template <int NW>
__device__ inline void block_min2_keys(uint32_t key, const FpsSmem& s, int& parity, uint32_t& k1, uint32_t& k2) {
  uint32_t a1 = key, a2 = 0xFFFFFFFFu;
  merge2(a1, a2, row_ror_u<8>(a1), row_ror_u<8>(a2));
  merge2(a1, a2, row_ror_u<4>(a1), row_ror_u<4>(a2));
  merge2(a1, a2, row_ror_u<2>(a1), row_ror_u<2>(a2));
  merge2(a1, a2, row_ror_u<1>(a1), row_ror_u<1>(a2));
  uint32_t w1 = (uint32_t)__builtin_amdgcn_readlane((int)a1, 0);
  uint32_t w2 = (uint32_t)__builtin_amdgcn_readlane((int)a2, 0);
  merge2(w1, w2, (uint32_t)__builtin_amdgcn_readlane((int)a1, 16), (uint32_t)__builtin_amdgcn_readlane((int)a2, 16));
  const int wave = threadIdx.x >> 6;
  uint32_t* slot = reinterpret_cast<uint32_t*>(s.islot) + parity * 2 * NW;
  if ((threadIdx.x & 63) == 0) {
    slot[2 * wave] = w1;
    slot[2 * wave + 1] = w2;
  }
  __syncthreads();
  k1 = slot[0];
  k2 = slot[1];
#pragma unroll
  for (int w = 1; w < NW; ++w) merge2(k1, k2, slot[2 * w], slot[2 * w + 1]);
  parity ^= 1;
}

// Matrix-core fragment of k-step `ks` for row `r` (bf16 32x32x16 takes dims
// 16 ks + 8 (lane / 32) + [0, 8); fp32 32x32x2 takes dim 2 ks + lane / 32).
template <int DT>
struct GramMma;

template <>
struct GramMma<BKV_BF16> {
  template <int D>
  static constexpr int steps() { return D / 16; }
  __device__ static inline fps_bf16x8 frag(const unsigned char* row, int ks, int lane) {
    uint4 w = *reinterpret_cast<const uint4*>(row + (size_t)(16 * ks + 8 * (lane >> 5)) * 2);
    return __builtin_bit_cast(fps_bf16x8, w);
  }
  __device__ static inline fps_floatx16 mma(fps_bf16x8 a, fps_bf16x8 b, fps_floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct GramMma<BKV_F32> {
  template <int D>
  static constexpr int steps() { return D / 2; }
  __device__ static inline float frag(const unsigned char* row, int ks, int lane) {
    return *reinterpret_cast<const float*>(row + (size_t)(2 * ks + (lane >> 5)) * 4);
  }
  __device__ static inline fps_floatx16 mma(float a, float b, fps_floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Binary64 decision among the candidates flagged `inwin` (row `myrow`):
// objective = mean cosine to all c rows (sum_mode) or maximum cosine to the
// picks so far (picks[0 .. npicked)).  Returns the row with the lowest
// objective, ties to the lower row.  Every thread of the block must call it.
// Wave w evaluates window members w, w + NW, ...; its lanes split the
// partner rows in groups of kP lanes (32 dimensions each).
template <int DT, int D, int NW>
__device__ int exact_window_argmin(const FpsSmem& s, bool inwin, int myrow, int c, int npicked, bool sum_mode,
                                   int& parity) {
  using F = Fps<DT, D, NW>;
  constexpr int kPerWave = 64 / F::kP;  // partner rows per sweep of a wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const double inf = __builtin_huge_val();
  int nu;
  const int pos = block_exclusive_scan(inwin ? 1 : 0, s.misc, &nu);
  if (inwin) s.ulist[pos] = myrow;
  __syncthreads();
  const int npart = sum_mode ? c : npicked;
  const int q = lane % F::kP;
  for (int u = wave; u < nu; u += NW) {
    const int a = s.ulist[u];
    double acc = sum_mode ? 0.0 : -inf;
    for (int j0 = 0; j0 < npart; j0 += kPerWave) {
      const int j = j0 + lane / F::kP;
      const int b = j < npart ? (sum_mode ? j : s.picks[j]) : a;
      double v = dot_slice64<DT, D, NW>(s, a, b, q);
      v = sum_lanes<F::kP>(v) * s.inv64[a] * s.inv64[b];
      if (j < npart) acc = sum_mode ? acc + v : fmax(acc, v);
    }
    // combine the partner groups of the wave (lanes 0, kP, 2 kP, ... hold them)
#pragma unroll
    for (int off = F::kP; off < 64; off <<= 1) {
      const double o = __shfl_xor(acc, off, 64);
      acc = sum_mode ? acc + o : fmax(acc, o);
    }
    if (lane == 0) s.uacc[u] = sum_mode ? acc / (double)c : acc;
  }
  __syncthreads();
  const bool in = tid < nu;
  return block_argmin64<NW>(in ? s.uacc[tid] : inf, in ? s.ulist[tid] : 0x7fffffff, s, parity);
}

// FPS over LDS rows [0, c), c <= 32 NW: writes min(k, c) picks to s.picks
// and returns the count.  Every thread of the block must call it; all 32 NW
// LDS rows must be readable.  Candidate row i is owned by lane i % 32 of wave
// i / 32, the wave whose MFMA accumulators hold Gram rows [32 w, 32 w + 32).
template <int DT, int D, int NW>
__device__ int fps_core(const FpsSmem& s, int c, int k) {
  using F = Fps<DT, D, NW>;
  using E = Elem<DT>;
  using MM = GramMma<DT>;
  constexpr int KS = MM::template steps<D>();
  const int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float finf = __builtin_huge_valf();
  int parity = 0;  // one toggle for every block reduction: consecutive reductions use different slots

  // 1. binary64 norms (clamped at 1e-12) and the fp32-safety check
  int unsafe = 0;
  if (tid < c) {
    const uint4* x = reinterpret_cast<const uint4*>(fps_row<DT, D, NW>(s, tid));
    double ss = 0.0;
#pragma unroll 2
    for (int u = 0; u < F::kU; ++u) {
      const uint4 w = x[u];
      const typename E::T* e = reinterpret_cast<const typename E::T*>(&w);
#pragma unroll
      for (int j = 0; j < F::kPer16; ++j) {
        const double v = E::to_f64(e[j]);
        ss = fma(v, v, ss);
      }
    }
    const double n = sqrt(ss);
    unsafe = (n > 0.0 && (n < 1e-15 || n > 1e18)) ? 1 : 0;
    const double inv = 1.0 / (n < 1e-12 ? 1e-12 : n);
    s.inv64[tid] = inv;
    s.inv32[tid] = (float)inv;
  }
  const bool unsafe_any = __syncthreads_or(unsafe) != 0;

  // candidate owned by this lane
  const int myrow = 32 * wave + (lane & 31);
  const bool owner = lane < 32 && myrow < c;

  if (unsafe_any) {  // plain binary64 rounds over every candidate
    int pick = exact_window_argmin<DT, D, NW>(s, owner, myrow, c, 0, true, parity);
    if (tid == 0) s.picks[0] = pick;
    bool picked = myrow == pick;
    for (int t = 1; t < kk; ++t) {
      __syncthreads();  // picks[t - 1] visible
      pick = exact_window_argmin<DT, D, NW>(s, owner && !picked, myrow, c, t, false, parity);
      if (myrow == pick) picked = true;
      if (tid == 0) s.picks[t] = pick;
    }
    __syncthreads();
    return kk;
  }

  // 2. Gram rows of this wave's tile on the matrix cores.  Every wave
  // multiplies every tile of the 32 NW LDS rows (rows at or beyond c hold
  // unused values): the MFMA chain is branch-free, so the compiler's
  // accumulator-read wait states cover every path to the reads below.
  fps_floatx16 acc[NW];
  {
    const unsigned char* arow = s.rows + (size_t)(32 * wave + (lane & 31)) * F::kRowStride;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const unsigned char* brow = s.rows + (size_t)(32 * t + (lane & 31)) * F::kRowStride;
      acc[t] = fps_floatx16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc[t] = MM::mma(MM::frag(arow, ks, lane), MM::frag(brow, ks, lane), acc[t]);
    }
  }
  float* colx = s.colx + 32 * wave;
  const int half = lane >> 5;
  const float inv_me = owner ? s.inv32[myrow] : 0.0f;

  // 3. start: lowest mean cosine; fp32 row sums of the normalised Gram, with
  // a binary64 decision when the best two are within the error window
  int pick;
  {
    float part[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = 0.0f;
#pragma unroll
    for (int t = 0; t < NW; ++t) {
      const int col = 32 * t + (lane & 31);
      const bool ok = col < c;
      const float w = ok ? s.inv32[col] : 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) part[r] += ok ? acc[t][r] * w : 0.0f;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) part[r] = half_wave_sum(part[r]);
    if ((lane & 31) == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) colx[8 * (r >> 2) + 4 * half + (r & 3)] = part[r];
    }
    __builtin_amdgcn_wave_barrier();
    const float mu = owner ? colx[lane & 31] * inv_me / (float)c : finf;
    __builtin_amdgcn_wave_barrier();
    uint32_t k1, k2;
    block_min2_keys<NW>(owner ? cand_key(mu, myrow) : 0xFFFFFFFFu, s, parity, k1, k2);
    const float eps_mu = F::kEps + 4.0f * (float)(c + 8) * F::kU32;
    const float hi1 = key_hi(k1) + 2.0f * eps_mu;
    if (k2 != 0xFFFFFFFFu && key_lo(k2) <= hi1) {
      const bool inwin = owner && mu <= hi1;
      pick = exact_window_argmin<DT, D, NW>(s, inwin, myrow, c, 0, true, parity);
    } else {
      pick = (int)(k1 & 0xFFu);
    }
  }
  if (tid == 0) s.picks[0] = pick;

  // 4. greedy rounds on fp32 cosines with the certified window
  const float eps2 = 2.0f * F::kEps;
  float mt = finf;  // max fp32 cosine of this candidate to the picked set
  bool picked = myrow == pick;
  for (int t = 1; t < kk; ++t) {
    // column `pick` of this wave's Gram tile, moved to the candidate owners
    {
      const int pt = pick >> 5;
      fps_floatx16 colv = acc[0];
#pragma unroll
      for (int tt = 1; tt < NW; ++tt)
        if (tt == pt) colv = acc[tt];
      if ((lane & 31) == (pick & 31)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) colx[8 * (r >> 2) + 4 * half + (r & 3)] = colv[r];
      }
    }
    __builtin_amdgcn_wave_barrier();
    const bool cand = owner && !picked;
    if (cand) {
      const float cv = colx[lane & 31] * inv_me * s.inv32[pick];
      mt = (t == 1) ? cv : fmaxf(mt, cv);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t k1, k2;
    block_min2_keys<NW>(cand ? cand_key(mt, myrow) : 0xFFFFFFFFu, s, parity, k1, k2);
    const float hi1 = key_hi(k1) + eps2;
    if (k2 != 0xFFFFFFFFu && key_lo(k2) <= hi1) {
      const bool inwin = cand && mt <= hi1;
      pick = exact_window_argmin<DT, D, NW>(s, inwin, myrow, c, t, false, parity);
    } else {
      pick = (int)(k1 & 0xFFu);
    }
    if (myrow == pick) picked = true;
    if (tid == 0) s.picks[t] = pick;
  }
  __syncthreads();
  return kk;
}

// ---------------------------------------------------------------------------
// Ingest
// ---------------------------------------------------------------------------

template <int DT, int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fps_update_kernel(const typename Elem<DT>::T* __restrict__ q_new, int T,
                                                             typename Elem<DT>::T* __restrict__ qbuf,
                                                             int32_t* __restrict__ qcount, int C, int M,
                                                             int32_t* __restrict__ ws_words) {
  using F = Fps<DT, D, NW>;
  using ET = typename F::ET;
  constexpr int NT = F::NT;
  constexpr int kU = F::kU;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
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
    copy16(buf + (size_t)c0 * D, qn, T * F::kRowBytes, tid, NT);
    if (tid == 0) qcount[head] = c0 + T;
    return;
  }
  constexpr int cpad = F::kMaxRows;  // rows [C, cpad) are readable padding, [cpad, cpad + M) the reorder area
  FpsSmem s = fps_carve<DT, D, NW>(smem, cpad + M);
  auto load_rows = [&](int dst_row, const ET* src, int nrows) {
    for (int u = tid; u < nrows * kU; u += NT) {
      const int r = u / kU, q = u % kU;
      reinterpret_cast<uint4*>(s.rows + (size_t)(dst_row + r) * F::kRowStride)[q] =
          reinterpret_cast<const uint4*>(src + (size_t)r * D)[q];
    }
  };
  load_rows(0, buf, c0);
  int c = c0;
  int t = 0;
  while (t < T) {
    const int take = (T - t) < (C - c) ? (T - t) : (C - c);
    load_rows(c, qn + (size_t)t * D, take);
    c += take;
    t += take;
    __syncthreads();
    if (c == C) {
      const int n = fps_core<DT, D, NW>(s, C, M);
      for (int u = tid; u < n * kU; u += NT) {
        const int r = u / kU, q = u % kU;
        reinterpret_cast<uint4*>(s.rows + (size_t)(cpad + r) * F::kRowStride)[q] =
            reinterpret_cast<const uint4*>(s.rows + (size_t)s.picks[r] * F::kRowStride)[q];
      }
      __syncthreads();
      for (int u = tid; u < n * kU; u += NT) {
        const int r = u / kU, q = u % kU;
        reinterpret_cast<uint4*>(s.rows + (size_t)r * F::kRowStride)[q] =
            reinterpret_cast<const uint4*>(s.rows + (size_t)(cpad + r) * F::kRowStride)[q];
      }
      __syncthreads();
      c = n;
    }
  }
  for (int u = tid; u < c * kU; u += NT) {
    const int r = u / kU, q = u % kU;
    reinterpret_cast<uint4*>(buf + (size_t)r * D)[q] =
        reinterpret_cast<const uint4*>(s.rows + (size_t)r * F::kRowStride)[q];
  }
  if (tid == 0) qcount[head] = c;
}

// ---------------------------------------------------------------------------
// RoPE tables: (cos, sin) per slot for the R recent positions and pos_now
// ---------------------------------------------------------------------------

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

// ---------------------------------------------------------------------------
// Observation rows: beacons (FPS over the buffer, rotated to pos_now) and
// recent queries (rotated to their own positions)
// ---------------------------------------------------------------------------

template <int DT, int D>
__device__ inline void rotate_store(const typename Elem<DT>::T* x, float2 cs, int i, typename Elem<DT>::T* y) {
  using E = Elem<DT>;
  constexpr int H = D / 2;
  // binary64 products of a storage value and a binary32 cos/sin are exact,
  // so each output is the correctly rounded binary64 value of the exact
  // rotation, rounded once more to the storage type
  const double x0 = E::to_f64(x[i]);
  const double x1 = E::to_f64(x[i + H]);
  const double c = (double)cs.x, s = (double)cs.y;
  y[i] = E::from_f64(x0 * c - x1 * s);
  y[i + H] = E::from_f64(x1 * c + x0 * s);
}

template <int DT, int D, int NW>
__global__ __launch_bounds__(64 * NW, 2) void obs_build_kernel(
    const typename Elem<DT>::T* __restrict__ qbuf, const int32_t* __restrict__ qcount, int C, int nb,
    const typename Elem<DT>::T* __restrict__ recent, const int32_t* __restrict__ recent_pos, int R,
    const float2* __restrict__ tab, typename Elem<DT>::T* __restrict__ obs, int32_t* __restrict__ obs_valid,
    int Hq, int Hkv, int RP, int32_t* __restrict__ ws_words) {
  using F = Fps<DT, D, NW>;
  using ET = typename F::ET;
  constexpr int NT = F::NT;
  constexpr int H = D / 2;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int head = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = head / Hq;
  const int gq = head % Hq;
  const int G = Hq / Hkv;
  const int h = gq / G;
  const int gl = gq % G;
  const size_t unit = (size_t)n * Hkv + h;
  const int rowbase = gl * (R + nb);
  ET* obs_u = obs + unit * RP * D;
  int32_t* val_u = obs_valid + unit * RP;
  const float2* tab_n = tab + (size_t)n * (R + 1) * H;

  // recent queries at their own positions
  for (int e = tid; e < R * H; e += NT) {
    const int r = e / H, i = e % H;
    ET* y = obs_u + (size_t)(rowbase + r) * D;
    if (recent_pos[(size_t)n * R + r] >= 0) {
      rotate_store<DT, D>(recent + ((size_t)head * R + r) * D, tab_n[r * H + i], i, y);
    } else {
      y[i] = ET(0);
      y[i + H] = ET(0);
    }
  }
  if (tid < R) val_u[rowbase + tid] = recent_pos[(size_t)n * R + tid] >= 0 ? 1 : 0;

  // beacons: FPS over the live buffer
  int c = qcount[head];
  if (c < 0 || c >= C) {
    if (tid == 0) set_status(ws_words, BKV_DEV_BAD_COUNT);
    c = 0;
  }
  const int want = nb < c ? nb : c;
  constexpr int cpad = F::kMaxRows;
  FpsSmem s = fps_carve<DT, D, NW>(smem, cpad);
  int kk = 0;
  if (want > 0) {
    const ET* buf = qbuf + (size_t)head * C * D;
    for (int u = tid; u < c * F::kU; u += NT) {
      const int r = u / F::kU, q = u % F::kU;
      reinterpret_cast<uint4*>(s.rows + (size_t)r * F::kRowStride)[q] =
          reinterpret_cast<const uint4*>(buf + (size_t)r * D)[q];
    }
    __syncthreads();
    kk = fps_core<DT, D, NW>(s, c, want);
  }
  for (int e = tid; e < nb * H; e += NT) {
    const int b = e / H, i = e % H;
    ET* y = obs_u + (size_t)(rowbase + R + b) * D;
    if (b < kk) {
      rotate_store<DT, D>(fps_row<DT, D, NW>(s, s.picks[b]), tab_n[R * H + i], i, y);
    } else {
      y[i] = ET(0);
      y[i + H] = ET(0);
    }
  }
  if (tid < nb) val_u[rowbase + R + tid] = tid < kk ? 1 : 0;

  // padding rows of the unit (written once, by the last query head of the group)
  if (gl == G - 1) {
    const int first = G * (R + nb);
    for (int e = tid; e < (RP - first) * D; e += NT) obs_u[(size_t)first * D + e] = ET(0);
    for (int r = first + tid; r < RP; r += NT) val_u[r] = 0;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers (block size from the capacity: 32 rows per wave)
// ---------------------------------------------------------------------------

template <int DT, int D, int NW>
static hipError_t launch_fps_update_nw(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M, int heads,
                                       int32_t* ws_words, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const int cpad = Fps<DT, D, NW>::kMaxRows;
  const size_t smem = fps_smem_bytes<DT, D, NW>(cpad + M);
  auto kern = fps_update_kernel<DT, D, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(64 * NW), smem, st, (const ET*)q_new, T, (ET*)qbuf, qcount, C, M,
                     ws_words);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_fps_update(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M, int heads,
                             int32_t* ws_words, hipStream_t st) {
  if (C <= 64) return launch_fps_update_nw<DT, D, 2>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
  if (C <= 128) return launch_fps_update_nw<DT, D, 4>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
  return launch_fps_update_nw<DT, D, 8>(q_new, T, qbuf, qcount, C, M, heads, ws_words, st);
}

template <int DT, int D, int NW>
static hipError_t launch_obs_nw(const void* qbuf, const int32_t* qcount, int C, int nb, const void* recent,
                                const int32_t* recent_pos, int R, float2* tab, void* obs, int32_t* obs_valid, int N,
                                int Hq, int Hkv, int RP, int32_t* ws_words, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const int cpad = Fps<DT, D, NW>::kMaxRows;
  const size_t smem = fps_smem_bytes<DT, D, NW>(cpad);
  auto kern = obs_build_kernel<DT, D, NW>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(N * Hq), dim3(64 * NW), smem, st, (const ET*)qbuf, qcount, C, nb, (const ET*)recent,
                     recent_pos, R, (const float2*)tab, (ET*)obs, obs_valid, Hq, Hkv, RP, ws_words);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_obs_build(const void* qbuf, const int32_t* qcount, int C, int nb, const void* recent,
                            const int32_t* recent_pos, int R, const int32_t* pos_now, double theta, float2* tab,
                            void* obs, int32_t* obs_valid, int N, int Hq, int Hkv, int RP, int32_t* ws_words,
                            hipStream_t st) {
  hipLaunchKernelGGL(rope_table_kernel<D>, dim3(N), dim3(256), 0, st, recent_pos, pos_now, R, theta, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (C <= 64)
    return launch_obs_nw<DT, D, 2>(qbuf, qcount, C, nb, recent, recent_pos, R, tab, obs, obs_valid, N, Hq, Hkv, RP,
                                   ws_words, st);
  if (C <= 128)
    return launch_obs_nw<DT, D, 4>(qbuf, qcount, C, nb, recent, recent_pos, R, tab, obs, obs_valid, N, Hq, Hkv, RP,
                                   ws_words, st);
  return launch_obs_nw<DT, D, 8>(qbuf, qcount, C, nb, recent, recent_pos, R, tab, obs, obs_valid, N, Hq, Hkv, RP,
                                 ws_words, st);
}

template hipError_t launch_fps_update<BKV_F32, 64>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                   hipStream_t);
template hipError_t launch_fps_update<BKV_F32, 128>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                    hipStream_t);
template hipError_t launch_fps_update<BKV_BF16, 64>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                    hipStream_t);
template hipError_t launch_fps_update<BKV_BF16, 128>(const void*, int, void*, int32_t*, int, int, int, int32_t*,
                                                     hipStream_t);
#define BKV_INST_OBS(DT, D)                                                                                    \
  template hipError_t launch_obs_build<DT, D>(const void*, const int32_t*, int, int, const void*,              \
                                              const int32_t*, int, const int32_t*, double, float2*, void*,     \
                                              int32_t*, int, int, int, int, int32_t*, hipStream_t);
BKV_INST_OBS(BKV_F32, 64)
BKV_INST_OBS(BKV_F32, 128)
BKV_INST_OBS(BKV_BF16, 64)
BKV_INST_OBS(BKV_BF16, 128)

}  // namespace bkv

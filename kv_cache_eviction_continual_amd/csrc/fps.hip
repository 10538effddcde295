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
// picked set; ties go to the lower row.  All cosines are evaluated in
// binary64 from the stored values (bf16 and fp32 widen exactly), so the
// argmin decisions are those of exact arithmetic up to binary64 rounding.
//
// Work split: one workgroup of 256 threads per query head.  The live buffer
// sits in LDS in its storage type (row stride padded by 16 bytes).  A
// candidate row is handled by P = d/32 adjacent lanes, each owning 32
// dimensions; a pick needs one 32-term binary64 dot product per owned
// candidate, a P-lane butterfly, a wave argmin and a cross-wave argmin
// through LDS (one barrier per pick).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

constexpr int kFpsThreads = 256;
constexpr int kFpsWaves = kFpsThreads / 64;

template <int DT, int D>
struct FpsLayout {
  using E = Elem<DT>;
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kRowStride = kRowBytes + 16;  // LDS padding against bank conflicts
  static constexpr int kP = D / 32;                  // lanes per candidate
  static constexpr int kGroups = kFpsThreads / kP;   // candidates handled per sweep
  static constexpr int kMaxOwn = (256 + kGroups - 1) / kGroups;  // C <= 256
};

// LDS carve-up shared by both kernels (C = capacity, M = extra rows).
struct FpsSmem {
  unsigned char* rows;  // [C + M] rows of kRowStride bytes
  double* inv_n;        // [256]
  double* svec;         // [D]
  double* part;         // [kFpsThreads] partial sums
  double* slot_v;       // [2][kFpsWaves]
  int* slot_i;          // [2][kFpsWaves]
  int* picks;           // [256]
};

template <int DT, int D>
__device__ inline FpsSmem carve(unsigned char* smem, int nrows) {
  using Lay = FpsLayout<DT, D>;
  FpsSmem s;
  size_t off = 0;
  s.rows = smem;
  off += (size_t)nrows * Lay::kRowStride;
  off = (off + 15) & ~(size_t)15;
  s.inv_n = reinterpret_cast<double*>(smem + off);
  off += 256 * sizeof(double);
  s.svec = reinterpret_cast<double*>(smem + off);
  off += D * sizeof(double);
  s.part = reinterpret_cast<double*>(smem + off);
  off += kFpsThreads * sizeof(double);
  s.slot_v = reinterpret_cast<double*>(smem + off);
  off += 2 * kFpsWaves * sizeof(double);
  s.slot_i = reinterpret_cast<int*>(smem + off);
  off += 2 * kFpsWaves * sizeof(int);
  s.picks = reinterpret_cast<int*>(smem + off);
  return s;
}

template <int DT, int D>
__host__ __device__ constexpr size_t fps_smem_bytes(int nrows) {
  return (((size_t)nrows * FpsLayout<DT, D>::kRowStride + 15) & ~(size_t)15) + 256 * sizeof(double) +
         D * sizeof(double) + kFpsThreads * sizeof(double) + 2 * kFpsWaves * (sizeof(double) + sizeof(int)) +
         256 * sizeof(int);
}

// Widen the 32-dimension slice `p` of LDS row `r` to binary64.
template <int DT, int D>
__device__ inline void load_slice(const FpsSmem& s, int r, int p, double (&x)[32]) {
  using Lay = FpsLayout<DT, D>;
  using E = Elem<DT>;
  const typename E::T* row =
      reinterpret_cast<const typename E::T*>(s.rows + (size_t)r * Lay::kRowStride) + p * 32;
  constexpr int kPer16 = 16 / E::kBytes;
#pragma unroll
  for (int q = 0; q < 32 / kPer16; ++q) {
    uint4 w = reinterpret_cast<const uint4*>(row)[q];
    const typename E::T* e = reinterpret_cast<const typename E::T*>(&w);
#pragma unroll
    for (int k = 0; k < kPer16; ++k) x[q * kPer16 + k] = E::to_f64(e[k]);
  }
}

template <int P>
__device__ inline double sum_over_p(double v) {
#pragma unroll
  for (int off = 1; off < P; off <<= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block-wide argmin of (value, index) with the strict order of `better`.
// Every thread passes its candidate; every thread receives the winner.
template <int P>
__device__ inline int block_argmin(double v, int i, const FpsSmem& s, int parity) {
#pragma unroll
  for (int off = P; off < 64; off <<= 1) {
    double ov = __shfl_xor(v, off, 64);
    int oi = __shfl_xor(i, off, 64);
    if (better(ov, oi, v, i)) {
      v = ov;
      i = oi;
    }
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s.slot_v[parity * kFpsWaves + wave] = v;
    s.slot_i[parity * kFpsWaves + wave] = i;
  }
  __syncthreads();
  double bv = s.slot_v[parity * kFpsWaves];
  int bi = s.slot_i[parity * kFpsWaves];
#pragma unroll
  for (int w = 1; w < kFpsWaves; ++w) {
    double ov = s.slot_v[parity * kFpsWaves + w];
    int oi = s.slot_i[parity * kFpsWaves + w];
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  return bi;
}

// FPS over LDS rows [0, c): writes min(k, c) picks to s.picks and returns the
// count.  All threads of the block must call it.
template <int DT, int D>
__device__ int fps_core(const FpsSmem& s, int c, int k) {
  using Lay = FpsLayout<DT, D>;
  using E = Elem<DT>;
  constexpr int P = Lay::kP;
  constexpr int NG = Lay::kGroups;
  constexpr int KO = Lay::kMaxOwn;
  const int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  const int tid = threadIdx.x;
  const int p = tid % P;
  const int cg = tid / P;
  const double inf = __builtin_huge_val();

  // 1. inverse norms of the owned candidates (norm clamped at 1e-12)
  double inv_n[KO];
  double m[KO];
  double x[32];
#pragma unroll
  for (int o = 0; o < KO; ++o) {
    const int i = cg + o * NG;
    inv_n[o] = 0.0;
    m[o] = inf;
    if (i < c) {
      load_slice<DT, D>(s, i, p, x);
      double ss = 0.0;
#pragma unroll
      for (int t = 0; t < 32; ++t) ss = fma(x[t], x[t], ss);
      ss = sum_over_p<P>(ss);
      double n = sqrt(ss);
      if (n < 1e-12) n = 1e-12;
      inv_n[o] = 1.0 / n;
      if (p == 0) s.inv_n[i] = inv_n[o];
    }
  }
  __syncthreads();

  // 2. sum of the normalised rows, svec = sum_i x_i / |x_i|
  {
    constexpr int kParts = kFpsThreads / D;
    const int dim = tid % D;
    const int part = tid / D;
    const typename E::T* col = nullptr;
    double acc = 0.0;
    for (int i = part; i < c; i += kParts) {
      col = reinterpret_cast<const typename E::T*>(s.rows + (size_t)i * Lay::kRowStride);
      acc = fma(E::to_f64(col[dim]), s.inv_n[i], acc);
    }
    s.part[tid] = acc;
    __syncthreads();
    if (tid < D) {
      double v = 0.0;
      for (int q = 0; q < kParts; ++q) v += s.part[q * D + tid];
      s.svec[tid] = v;
    }
    __syncthreads();
  }

  // 3. start: lowest mean cosine, mu_i = (x_i . svec) / (|x_i| c)
  int parity = 0;
  int start;
  {
    double sv[32];
#pragma unroll
    for (int t = 0; t < 32; ++t) sv[t] = s.svec[p * 32 + t];
    double bv = inf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      const int i = cg + o * NG;
      if (i < c) {
        load_slice<DT, D>(s, i, p, x);
        double dd = 0.0;
#pragma unroll
        for (int t = 0; t < 32; ++t) dd = fma(x[t], sv[t], dd);
        dd = sum_over_p<P>(dd);
        const double mu = dd * inv_n[o] / (double)c;
        if (better(mu, i, bv, bi)) {
          bv = mu;
          bi = i;
        }
      }
    }
    start = block_argmin<P>(bv, bi, s, parity);
    parity ^= 1;
  }
  if (tid == 0) s.picks[0] = start;

  // 4. greedy rounds; round 0 initialises m with the cosines to the start
  int pick = start;
  for (int t = 0; t < kk; ++t) {
    double xp[32];
    load_slice<DT, D>(s, pick, p, xp);
    const double inv_p = s.inv_n[pick];
    double bv = inf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int o = 0; o < KO; ++o) {
      const int i = cg + o * NG;
      if (i < c) {
        load_slice<DT, D>(s, i, p, x);
        double dd = 0.0;
#pragma unroll
        for (int q = 0; q < 32; ++q) dd = fma(x[q], xp[q], dd);
        dd = sum_over_p<P>(dd);
        const double cosv = dd * inv_n[o] * inv_p;
        if (i == pick) {
          m[o] = inf;  // picked rows leave the candidate set for good
        } else if (t == 0) {
          m[o] = cosv;
        } else if (m[o] != inf && cosv > m[o]) {
          m[o] = cosv;
        }
        if (better(m[o], i, bv, bi)) {
          bv = m[o];
          bi = i;
        }
      }
    }
    if (t + 1 == kk) break;
    pick = block_argmin<P>(bv, bi, s, parity);
    parity ^= 1;
    if (tid == 0) s.picks[t + 1] = pick;
  }
  __syncthreads();
  return kk;
}

// ---------------------------------------------------------------------------
// Ingest
// ---------------------------------------------------------------------------

template <int DT, int D>
__global__ __launch_bounds__(kFpsThreads) void fps_update_kernel(const typename Elem<DT>::T* __restrict__ q_new,
                                                                 int T, typename Elem<DT>::T* __restrict__ qbuf,
                                                                 int32_t* __restrict__ qcount, int C, int M,
                                                                 int32_t* __restrict__ ws_words) {
  using Lay = FpsLayout<DT, D>;
  using ET = typename Elem<DT>::T;
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
    copy16(buf + (size_t)c0 * D, qn, T * Lay::kRowBytes, tid, kFpsThreads);
    if (tid == 0) qcount[head] = c0 + T;
    return;
  }
  FpsSmem s = carve<DT, D>(smem, C + M);
  constexpr int kU = Lay::kRowBytes / 16;  // 16-byte units per row
  auto load_rows = [&](int dst_row, const ET* src, int nrows) {
    for (int u = tid; u < nrows * kU; u += kFpsThreads) {
      const int r = u / kU, q = u % kU;
      reinterpret_cast<uint4*>(s.rows + (size_t)(dst_row + r) * Lay::kRowStride)[q] =
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
      const int n = fps_core<DT, D>(s, C, M);
      // gather the picks, in pick order, through the spare rows [C, C+M)
      for (int u = tid; u < n * kU; u += kFpsThreads) {
        const int r = u / kU, q = u % kU;
        reinterpret_cast<uint4*>(s.rows + (size_t)(C + r) * Lay::kRowStride)[q] =
            reinterpret_cast<const uint4*>(s.rows + (size_t)s.picks[r] * Lay::kRowStride)[q];
      }
      __syncthreads();
      for (int u = tid; u < n * kU; u += kFpsThreads) {
        const int r = u / kU, q = u % kU;
        reinterpret_cast<uint4*>(s.rows + (size_t)r * Lay::kRowStride)[q] =
            reinterpret_cast<const uint4*>(s.rows + (size_t)(C + r) * Lay::kRowStride)[q];
      }
      __syncthreads();
      c = n;
    }
  }
  for (int u = tid; u < c * kU; u += kFpsThreads) {
    const int r = u / kU, q = u % kU;
    reinterpret_cast<uint4*>(buf + (size_t)r * D)[q] =
        reinterpret_cast<const uint4*>(s.rows + (size_t)r * Lay::kRowStride)[q];
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

template <int DT, int D>
__global__ __launch_bounds__(kFpsThreads) void obs_build_kernel(
    const typename Elem<DT>::T* __restrict__ qbuf, const int32_t* __restrict__ qcount, int C, int nb,
    const typename Elem<DT>::T* __restrict__ recent, const int32_t* __restrict__ recent_pos, int R,
    const float2* __restrict__ tab, typename Elem<DT>::T* __restrict__ obs, int32_t* __restrict__ obs_valid,
    int Hq, int Hkv, int RP, int32_t* __restrict__ ws_words) {
  using Lay = FpsLayout<DT, D>;
  using ET = typename Elem<DT>::T;
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
  for (int e = tid; e < R * H; e += kFpsThreads) {
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
  FpsSmem s = carve<DT, D>(smem, C);
  int kk = 0;
  if (want > 0) {
    const ET* buf = qbuf + (size_t)head * C * D;
    constexpr int kU = Lay::kRowBytes / 16;
    for (int u = tid; u < c * kU; u += kFpsThreads) {
      const int r = u / kU, q = u % kU;
      reinterpret_cast<uint4*>(s.rows + (size_t)r * Lay::kRowStride)[q] =
          reinterpret_cast<const uint4*>(buf + (size_t)r * D)[q];
    }
    __syncthreads();
    kk = fps_core<DT, D>(s, c, want);
  }
  for (int e = tid; e < nb * H; e += kFpsThreads) {
    const int b = e / H, i = e % H;
    ET* y = obs_u + (size_t)(rowbase + R + b) * D;
    if (b < kk) {
      const ET* x = reinterpret_cast<const ET*>(s.rows + (size_t)s.picks[b] * Lay::kRowStride);
      rotate_store<DT, D>(x, tab_n[R * H + i], i, y);
    } else {
      y[i] = ET(0);
      y[i + H] = ET(0);
    }
  }
  if (tid < nb) val_u[rowbase + R + tid] = tid < kk ? 1 : 0;

  // padding rows of the unit (written once, by the last query head of the group)
  if (gl == G - 1) {
    const int first = G * (R + nb);
    for (int e = tid; e < (RP - first) * D; e += kFpsThreads) obs_u[(size_t)first * D + e] = ET(0);
    for (int r = first + tid; r < RP; r += kFpsThreads) val_u[r] = 0;
  }
}

// ---------------------------------------------------------------------------
// Host-side launchers
// ---------------------------------------------------------------------------

template <int DT, int D>
hipError_t launch_fps_update(const void* q_new, int T, void* qbuf, int32_t* qcount, int C, int M, int heads,
                             int32_t* ws_words, hipStream_t st) {
  using ET = typename Elem<DT>::T;
  const size_t smem = fps_smem_bytes<DT, D>(C + M);
  auto kern = fps_update_kernel<DT, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(heads), dim3(kFpsThreads), smem, st, (const ET*)q_new, T, (ET*)qbuf, qcount, C, M,
                     ws_words);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_obs_build(const void* qbuf, const int32_t* qcount, int C, int nb, const void* recent,
                            const int32_t* recent_pos, int R, const int32_t* pos_now, double theta, float2* tab,
                            void* obs, int32_t* obs_valid, int N, int Hq, int Hkv, int RP, int32_t* ws_words,
                            hipStream_t st) {
  using ET = typename Elem<DT>::T;
  hipLaunchKernelGGL(rope_table_kernel<D>, dim3(N), dim3(256), 0, st, recent_pos, pos_now, R, theta, tab);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t smem = fps_smem_bytes<DT, D>(C);
  auto kern = obs_build_kernel<DT, D>;
  e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(N * Hq), dim3(kFpsThreads), smem, st, (const ET*)qbuf, qcount, C, nb,
                     (const ET*)recent, recent_pos, R, (const float2*)tab, (ET*)obs, obs_valid, Hq, Hkv, RP,
                     ws_words);
  return hipGetLastError();
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

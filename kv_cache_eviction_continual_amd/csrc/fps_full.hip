// fps_full.hip -- farthest point sampling over each query head's whole stored
// history: the naive alternative that Continual FPS replaces.  Running FPS
// over every query seen so far means keeping the full history of every head;
// the bounded, repeatedly compressed buffer exists to avoid exactly that
// (wzjinhao.cn news article 56682 on BeaconKV, section 怎么挑出这几个信标).
//
// The picking rule is the buffer FPS's: start at the row with the lowest mean
// cosine to all rows (itself included), then repeatedly add the unpicked row
// with the lowest maximum cosine to the picked rows; ties go to the lower row;
// norms are clamped at 1e-12.  The mean cosine of row i is taken as
// x_i . s / (|x_i| n) with s the sum of the normalised rows, which equals the
// pairwise mean by linearity.
//
// A history of tens of thousands of rows per head does not fit on chip, so
// every pick streams the head's rows from HBM once: the path is bound by that
// stream, and the arithmetic runs in binary64, which it hides.  One launch per
// step, each over (head, chunk of kChunk rows) workgroups:
//   sum_kernel    row norms (kept in the workspace) and per-chunk sums of the
//                 normalised rows;
//   start_kernel  every row's mean cosine; per-chunk minimum;
//   round_kernel  takes the previous step's minimum over the head's chunks as
//                 the next pick, then raises every row's maximum cosine by its
//                 cosine to that pick (picked rows get +inf); per-chunk
//                 minimum;
//   last_kernel   the last pick, and -1 for picks beyond the history.
// The per-chunk minima pass from one launch to the next through the
// workspace; stream order is the only synchronisation.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

constexpr int kFullChunk = 1024;                      // rows per workgroup
constexpr int kFullThreads = 256;                     // four waves
constexpr int kFullWaveRows = kFullChunk / (kFullThreads / 64);
constexpr int kFullUnroll = 8;                        // 4-row steps in flight per wave

struct FullCand {
  double v;
  int32_t i;
  int32_t pad;
};

struct U32x8 {
  uint4 a, b;
};

template <int BYTES>
struct RawOf;
template <>
struct RawOf<8> {
  using type = uint2;
};
template <>
struct RawOf<16> {
  using type = uint4;
};
template <>
struct RawOf<32> {
  using type = U32x8;
};

// Sixteen lanes share a row: lane part p holds elements [p EL, p EL + EL).
template <int DT, int D>
struct FullPart {
  using E = Elem<DT>;
  using T = typename E::T;
  static constexpr int EL = D / 16;
  using R = typename RawOf<EL * (int)sizeof(T)>::type;
  struct Arr {
    T e[EL];
  };
  __device__ static inline R load(const T* row, int part) { return *reinterpret_cast<const R*>(row + part * EL); }
  __device__ static inline void widen(const R& r, double (&x)[EL]) {
    const Arr a = __builtin_bit_cast(Arr, r);
#pragma unroll
    for (int k = 0; k < EL; ++k) x[k] = E::to_f64(a.e[k]);
  }
};

__device__ inline double sum16(double v) {
  v += __shfl_xor(v, 8, 16);
  v += __shfl_xor(v, 4, 16);
  v += __shfl_xor(v, 2, 16);
  v += __shfl_xor(v, 1, 16);
  return v;
}

// dots[r] = x_r . y for the chunk's rows r (rows at or beyond n are skipped);
// y is this lane's part of the other vector.
template <int DT, int D>
__device__ inline void chunk_dots(const typename Elem<DT>::T* X, long n, long c0, const double (&y)[D / 16],
                                  double* dots) {
  using P = FullPart<DT, D>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = lane & 15, sub = lane >> 4;
  const long w0 = c0 + (long)wave * kFullWaveRows;
  for (int s0 = 0; s0 < kFullWaveRows / 4; s0 += kFullUnroll) {
    typename P::R raw[kFullUnroll];
#pragma unroll
    for (int u = 0; u < kFullUnroll; ++u) {
      const long i = w0 + (s0 + u) * 4 + sub;
      if (i < n) raw[u] = P::load(X + i * D, part);
    }
#pragma unroll
    for (int u = 0; u < kFullUnroll; ++u) {
      const long i = w0 + (s0 + u) * 4 + sub;
      double x[P::EL];
      double acc = 0.0;
      if (i < n) {
        P::widen(raw[u], x);
#pragma unroll
        for (int k = 0; k < P::EL; ++k) acc = fma(x[k], y[k], acc);
      }
      acc = sum16(acc);
      if (part == 0 && i < n) dots[i - c0] = acc;
    }
  }
}

// Block argmin of (v, i) over the threads' candidates; thread 0 writes it.
__device__ inline void block_argmin_store(double bv, int bi, FullCand* out, double* sv, int* si) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const double ov = __shfl_xor(bv, off, 64);
    const int oi = __shfl_xor(bi, off, 64);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    sv[wave] = bv;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kFullThreads / 64; ++w)
      if (better(sv[w], si[w], bv, bi)) {
        bv = sv[w];
        bi = si[w];
      }
    out->v = bv;
    out->i = bi;
  }
}

// The head's best candidate over its chunks' minima (wave 0 reduces, the
// result goes to every thread through LDS).  With finite rows a finite
// candidate always exists; the clamp keeps the index inside the history if
// non-finite rows leave none (the picks are then unspecified).
__device__ inline int head_pick(const FullCand* cand, int nchunks, long n, int* sp) {
  if (threadIdx.x < 64) {
    double bv = INFINITY;
    int bi = INT32_MAX;
    for (int c = threadIdx.x; c < nchunks; c += 64) {
      const FullCand x = cand[c];
      if (better(x.v, x.i, bv, bi)) {
        bv = x.v;
        bi = x.i;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const double ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if (threadIdx.x == 0) *sp = (bi >= 0 && bi < n) ? bi : (int)(n - 1);
  }
  __syncthreads();
  return *sp;
}

template <int DT, int D>
__global__ __launch_bounds__(kFullThreads) void fps_full_sum_kernel(const void* __restrict__ hist, long n,
                                                                    int nchunks, double* __restrict__ nrm,
                                                                    double* __restrict__ partial) {
  using P = FullPart<DT, D>;
  using T = typename Elem<DT>::T;
  __shared__ double red[kFullThreads / 64][D];
  const long head = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const T* X = reinterpret_cast<const T*>(hist) + head * n * D;
  double* nh = nrm + head * n;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int part = lane & 15, sub = lane >> 4;
  const long w0 = (long)chunk * kFullChunk + (long)wave * kFullWaveRows;
  double acc[P::EL];
#pragma unroll
  for (int k = 0; k < P::EL; ++k) acc[k] = 0.0;
  for (int s0 = 0; s0 < kFullWaveRows / 4; s0 += kFullUnroll) {
    typename P::R raw[kFullUnroll];
#pragma unroll
    for (int u = 0; u < kFullUnroll; ++u) {
      const long i = w0 + (s0 + u) * 4 + sub;
      if (i < n) raw[u] = P::load(X + i * D, part);
    }
#pragma unroll
    for (int u = 0; u < kFullUnroll; ++u) {
      const long i = w0 + (s0 + u) * 4 + sub;
      double x[P::EL];
      double ss = 0.0;
      if (i < n) {
        P::widen(raw[u], x);
#pragma unroll
        for (int k = 0; k < P::EL; ++k) ss = fma(x[k], x[k], ss);
      }
      ss = sum16(ss);
      const double r = fmax(sqrt(ss), 1e-12);
      if (i < n) {
        if (part == 0) nh[i] = r;
        const double ir = 1.0 / r;  // one division per row; the sum's order differs from the oracle's anyway
#pragma unroll
        for (int k = 0; k < P::EL; ++k) acc[k] = fma(x[k], ir, acc[k]);
      }
    }
  }
  // combine the four row groups of the wave, then the four waves
#pragma unroll
  for (int k = 0; k < P::EL; ++k) {
    acc[k] += __shfl_xor(acc[k], 16, 64);
    acc[k] += __shfl_xor(acc[k], 32, 64);
  }
  if (sub == 0) {
#pragma unroll
    for (int k = 0; k < P::EL; ++k) red[wave][part * P::EL + k] = acc[k];
  }
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int w = 0; w < kFullThreads / 64; ++w) s += red[w][threadIdx.x];
    partial[((long)head * nchunks + chunk) * D + threadIdx.x] = s;
  }
}

template <int DT, int D>
__global__ __launch_bounds__(kFullThreads) void fps_full_start_kernel(const void* __restrict__ hist, long n,
                                                                      int nchunks, const double* __restrict__ nrm,
                                                                      const double* __restrict__ partial,
                                                                      FullCand* __restrict__ cand) {
  using T = typename Elem<DT>::T;
  constexpr int EL = D / 16;
  __shared__ double dots[kFullChunk];
  __shared__ double s[D];
  __shared__ double sv[kFullThreads / 64];
  __shared__ int si[kFullThreads / 64];
  const long head = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const long c0 = (long)chunk * kFullChunk;
  if (threadIdx.x < D) {
    double a = 0.0;
    for (int c = 0; c < nchunks; ++c) a += partial[((long)head * nchunks + c) * D + threadIdx.x];
    s[threadIdx.x] = a;
  }
  __syncthreads();
  double y[EL];
  const int part = threadIdx.x & 15;
#pragma unroll
  for (int k = 0; k < EL; ++k) y[k] = s[part * EL + k];
  chunk_dots<DT, D>(reinterpret_cast<const T*>(hist) + head * n * D, n, c0, y, dots);
  __syncthreads();
  double bv = INFINITY;
  int bi = INT32_MAX;
  const double* nh = nrm + head * n;
  for (int r = threadIdx.x; r < kFullChunk; r += kFullThreads) {
    const long i = c0 + r;
    if (i >= n) break;
    const double mu = dots[r] / nh[i] / (double)n;
    if (better(mu, (int)i, bv, bi)) {
      bv = mu;
      bi = (int)i;
    }
  }
  block_argmin_store(bv, bi, cand + head * nchunks + chunk, sv, si);
}

template <int DT, int D>
__global__ __launch_bounds__(kFullThreads) void fps_full_round_kernel(const void* __restrict__ hist, long n,
                                                                      int nchunks, const double* __restrict__ nrm,
                                                                      double* __restrict__ m, int first,
                                                                      const FullCand* __restrict__ prev,
                                                                      FullCand* __restrict__ next,
                                                                      int32_t* __restrict__ picks, int k, int slot) {
  using T = typename Elem<DT>::T;
  using P = FullPart<DT, D>;
  constexpr int EL = D / 16;
  __shared__ double dots[kFullChunk];
  __shared__ double sv[kFullThreads / 64];
  __shared__ int si[kFullThreads / 64];
  __shared__ int sp;
  const long head = blockIdx.x / nchunks;
  const int chunk = blockIdx.x % nchunks;
  const long c0 = (long)chunk * kFullChunk;
  const int p = head_pick(prev + head * nchunks, nchunks, n, &sp);
  if (chunk == 0 && threadIdx.x == 0) picks[head * k + slot] = p;
  const T* X = reinterpret_cast<const T*>(hist) + head * n * D;
  double y[EL];
  P::widen(P::load(X + (long)p * D, threadIdx.x & 15), y);
  chunk_dots<DT, D>(X, n, c0, y, dots);
  __syncthreads();
  const double* nh = nrm + head * n;
  double* mh = m + head * n;
  const double np_ = nh[p];
  double bv = INFINITY;
  int bi = INT32_MAX;
  for (int r = threadIdx.x; r < kFullChunk; r += kFullThreads) {
    const long i = c0 + r;
    if (i >= n) break;
    const double cs = dots[r] / (nh[i] * np_);
    double v = first ? cs : fmax(mh[i], cs);
    if (i == p) v = INFINITY;
    mh[i] = v;
    if (v != INFINITY && better(v, (int)i, bv, bi)) {
      bv = v;
      bi = (int)i;
    }
  }
  block_argmin_store(bv, bi, next + head * nchunks + chunk, sv, si);
}

__global__ void fps_full_last_kernel(long n, int nchunks, const FullCand* __restrict__ prev,
                                     int32_t* __restrict__ picks, int k, int kk) {
  __shared__ int sp;
  const long head = blockIdx.x;
  int p = -1;
  if (kk > 0) p = head_pick(prev + head * nchunks, nchunks, n, &sp);
  for (int t = threadIdx.x; t < k; t += blockDim.x) {
    if (t == kk - 1) picks[head * k + t] = p;
    else if (t >= kk) picks[head * k + t] = -1;
  }
}

size_t fps_full_workspace_bytes(long heads, long n, int d) {
  const long nchunks = (n + kFullChunk - 1) / kFullChunk;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al(sizeof(double) * heads * n) * 2 + al(sizeof(double) * heads * nchunks * d) +
         al(sizeof(FullCand) * heads * nchunks) * 2;
}

template <int DT, int D>
hipError_t launch_fps_full(const void* hist, long heads, long n, int k, int32_t* picks, void* ws, hipStream_t st) {
  const int kk = (int)(k < n ? k : n);
  const int nchunks = (int)((n + kFullChunk - 1) / kFullChunk);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  unsigned char* b = reinterpret_cast<unsigned char*>(ws);
  double* nrm = reinterpret_cast<double*>(b);
  b += al(sizeof(double) * heads * n);
  double* m = reinterpret_cast<double*>(b);
  b += al(sizeof(double) * heads * n);
  double* partial = reinterpret_cast<double*>(b);
  b += al(sizeof(double) * heads * nchunks * D);
  FullCand* cand[2];
  cand[0] = reinterpret_cast<FullCand*>(b);
  b += al(sizeof(FullCand) * heads * nchunks);
  cand[1] = reinterpret_cast<FullCand*>(b);
  if (kk > 0) {
    const unsigned grid = (unsigned)(heads * nchunks);
    fps_full_sum_kernel<DT, D><<<grid, kFullThreads, 0, st>>>(hist, n, nchunks, nrm, partial);
    fps_full_start_kernel<DT, D><<<grid, kFullThreads, 0, st>>>(hist, n, nchunks, nrm, partial, cand[0]);
    for (int j = 1; j < kk; ++j)
      fps_full_round_kernel<DT, D><<<grid, kFullThreads, 0, st>>>(hist, n, nchunks, nrm, m, j == 1,
                                                                  cand[(j - 1) & 1], cand[j & 1], picks, k, j - 1);
  }
  if (k > 0) fps_full_last_kernel<<<(unsigned)heads, 64, 0, st>>>(n, nchunks, cand[(kk - 1 + 2) & 1], picks, k, kk);
  return hipGetLastError();
}

template hipError_t launch_fps_full<BKV_BF16, 128>(const void*, long, long, int, int32_t*, void*, hipStream_t);
template hipError_t launch_fps_full<BKV_BF16, 64>(const void*, long, long, int, int32_t*, void*, hipStream_t);
template hipError_t launch_fps_full<BKV_F32, 128>(const void*, long, long, int, int32_t*, void*, hipStream_t);
template hipError_t launch_fps_full<BKV_F32, 64>(const void*, long, long, int, int32_t*, void*, hipStream_t);

}  // namespace bkv

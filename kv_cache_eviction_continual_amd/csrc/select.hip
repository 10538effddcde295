// select.hip -- top-B_KV selection with an always-kept window, and in-place
// order-preserving compaction of K and V, on gfx950.
//
// Selection (inkeast.github.io MessageDaily paper-reading post on BeaconKV,
// section 三: I = TopK(score(K,V), B_KV); aimodeling.com "BeaconKV: Beacon
// Queries Fix KV Eviction for Long Reasoning", section "Beacon queries
// anticipate what will be revisited": the recent sliding window is always
// kept).  B_KV counts the window; the other B_KV - W entries are the highest
// scores of [0, L - W), ties at the cut going to the lower index.
//
// select_kernel: one workgroup per (slot, KV head).  Scores are non-negative
// floats, so their bit patterns order like the values; an MSB-first radix
// select (4 passes of 8 bits, LDS histograms) finds the cut value tau and
// how many entries equal to tau are taken.  One more pass marks the kept
// entries in index order (block prefix sums) and writes them ascending.
//
// compact_kernel: one workgroup per (slot, KV head, tensor).  Row i <- row
// kept[i] for i from the first evicted index up to the kept count.  Because
// kept is ascending, kept[i] >= i: a row is only ever read by a destination
// at or before its own index.  Rows move in steps of increasing index; a
// block-wide barrier after each step's loads have returned orders every read
// of a row before its overwrite.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bkv_device.hpp"

namespace bkv {

constexpr int kSelThreads = 256;

__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ len, int Hkv, int Lmax,
                                                             int B, int W, int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ sel,
                                                             int32_t* __restrict__ ws_words) {
  __shared__ int hist[256];
  __shared__ int scan_tmp[16];
  __shared__ int bcast[4];
  const size_t unit = blockIdx.x;
  const int n = (int)(unit / Hkv);
  const int tid = threadIdx.x;
  const int L = len[n];
  int32_t* kept_u = kept + unit * (size_t)B;
  if (L < 0 || L > Lmax) {
    if (tid == 0) {
      set_status(ws_words, BKV_DEV_BAD_LEN);
      sel[2 * unit] = 0;
      sel[2 * unit + 1] = -1;  // compaction skips the unit
    }
    return;
  }
  if (L <= B) {  // nothing to evict
    for (int i = tid; i < B; i += kSelThreads) kept_u[i] = i < L ? i : -1;
    if (tid == 0) {
      sel[2 * unit] = L;
      sel[2 * unit + 1] = L;
    }
    return;
  }
  const uint32_t* u = reinterpret_cast<const uint32_t*>(scores + unit * (size_t)Lmax);
  const int ncand = L - W;  // candidates [0, L - W)
  const int want = B - W;   // how many candidates survive

  // radix select of the want-th largest bit pattern among the candidates
  uint32_t prefix = 0, mask = 0;
  int remaining = want;  // entries still to take at or below the current prefix
  if (want > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
      __syncthreads();
      for (int j = tid; j < ncand; j += kSelThreads) {
        const uint32_t x = u[j];
        if ((x & mask) == prefix) atomicAdd(&hist[(x >> shift) & 255], 1);
      }
      __syncthreads();
      // suffix sums from the top bucket: thread t owns bucket 255 - t
      const int b = 255 - tid;
      int cnt = tid < 256 ? hist[b] : 0;
      int total;
      const int above = block_exclusive_scan(cnt, scan_tmp, &total);  // entries in buckets > b
      if (tid < 256 && above < remaining && remaining <= above + cnt) {
        bcast[0] = b;
        bcast[1] = remaining - above;
      }
      __syncthreads();
      prefix |= (uint32_t)bcast[0] << shift;
      mask |= 255u << shift;
      remaining = bcast[1];
      __syncthreads();
    }
  }
  const uint32_t tau = prefix;  // exact bit pattern of the cut value
  const int take_eq = remaining; // entries equal to tau to keep, lowest index first

  // mark and write: kept = (x > tau) or (x == tau and among the first take_eq
  // equal entries) over the candidates, plus the window
  int eq_base = 0, out_base = 0;
  int first_hole = 0x7fffffff;
  for (int j0 = 0; j0 < L; j0 += kSelThreads) {
    const int j = j0 + tid;
    bool gt = false, eq = false, win = false;
    if (j < ncand) {
      if (want > 0) {
        const uint32_t x = u[j];
        gt = x > tau;
        eq = x == tau;
      }
    } else if (j < L) {
      win = true;
    }
    int eq_total;
    const int eq_rank = block_exclusive_scan(eq ? 1 : 0, scan_tmp, &eq_total);
    const bool keep = gt || win || (eq && eq_base + eq_rank < take_eq);
    int keep_total;
    const int pos = block_exclusive_scan(keep ? 1 : 0, scan_tmp, &keep_total);
    if (keep) kept_u[out_base + pos] = j;
    if (j < L && !keep && j < first_hole) first_hole = j;
    eq_base += eq_total;
    out_base += keep_total;
  }
  // block minimum of first_hole
  for (int off = 32; off > 0; off >>= 1) {
    int o = __shfl_xor(first_hole, off, 64);
    first_hole = o < first_hole ? o : first_hole;
  }
  if ((tid & 63) == 0) scan_tmp[tid >> 6] = first_hole;
  __syncthreads();
  if (tid == 0) {
    int f = scan_tmp[0];
    for (int w = 1; w < kSelThreads / 64; ++w) f = scan_tmp[w] < f ? scan_tmp[w] : f;
    sel[2 * unit] = f < B ? f : B;
    sel[2 * unit + 1] = B;
  }
}

// ---------------------------------------------------------------------------

constexpr int kCompactThreads = 256;

// Row data is streamed once: non-temporal 16-byte loads and stores (measured
// ~5-10 % above plain ones for large copies on this part).
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline nt_u32x4 nt_load16(const unsigned char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
}
__device__ inline void nt_store16(unsigned char* p, nt_u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<nt_u32x4*>(p));
}
constexpr int kCompactUnroll = 2;  // row groups per thread per step (more in flight measured slower)

// One workgroup per (slot, KV head, tensor).  A step moves kCompactUnroll
// groups of (256 / lanes per row) rows: every thread first waits for its own
// loads and stores, the block synchronises, then the loads of the next step
// are issued (they read rows at or beyond the next step's first index, which
// this step's stores never touch) followed by this step's stores (whose rows
// are read only by destinations at or before them, all loaded already).
__global__ __launch_bounds__(kCompactThreads) void compact_kernel(unsigned char* __restrict__ K,
                                                                  unsigned char* __restrict__ V,
                                                                  const int32_t* __restrict__ kept,
                                                                  const int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ len, int Hkv, int Lmax, int B,
                                                                  int row_bytes,
                                                                  unsigned long long* __restrict__ rows_moved) {
  const size_t unit = blockIdx.x >> 1;
  const int tensor = blockIdx.x & 1;
  const int tid = threadIdx.x;
  const int f = sel[2 * unit];
  const int cnt = sel[2 * unit + 1];
  if (cnt < 0) return;  // unit rejected by the selection
  const int n = (int)(unit / Hkv);
  if (tid == 0) {
    if (tensor == 0 && unit % Hkv == 0) len[n] = cnt;  // no compaction block reads len
    if (cnt > f) atomicAdd(rows_moved, (unsigned long long)(cnt - f));
  }
  if (cnt <= f) return;
  unsigned char* base = (tensor ? V : K) + unit * (size_t)Lmax * row_bytes;
  const int32_t* kept_u = kept + unit * (size_t)B;
  const int lanes_per_row = row_bytes / 16;
  const int rows_per_group = kCompactThreads / lanes_per_row;
  const int col = (tid % lanes_per_row) * 16;
  const int sub = tid / lanes_per_row;
  const int rows_per_step = rows_per_group * kCompactUnroll;

  nt_u32x4 cur[kCompactUnroll], nxt[kCompactUnroll];
#pragma unroll
  for (int k = 0; k < kCompactUnroll; ++k) {
    const int i = f + k * rows_per_group + sub;
    if (i < cnt) cur[k] = nt_load16(base + (size_t)kept_u[i] * row_bytes + col);
  }
  for (int i0 = f; i0 < cnt; i0 += rows_per_step) {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int nx = i0 + rows_per_step;
    if (nx < cnt) {
#pragma unroll
      for (int k = 0; k < kCompactUnroll; ++k) {
        const int i = nx + k * rows_per_group + sub;
        if (i < cnt) nxt[k] = nt_load16(base + (size_t)kept_u[i] * row_bytes + col);
      }
    }
#pragma unroll
    for (int k = 0; k < kCompactUnroll; ++k) {
      const int i = i0 + k * rows_per_group + sub;
      if (i < cnt) nt_store16(base + (size_t)i * row_bytes + col, cur[k]);
    }
#pragma unroll
    for (int k = 0; k < kCompactUnroll; ++k) cur[k] = nxt[k];
  }
}

hipError_t launch_select(const float* scores, const int32_t* len, int N, int Hkv, int Lmax, int B, int W,
                         int32_t* kept, int32_t* sel, int32_t* ws_words, hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(N * Hkv), dim3(kSelThreads), 0, st, scores, len, Hkv, Lmax, B, W, kept, sel,
                     ws_words);
  return hipGetLastError();
}

hipError_t launch_compact(void* K, void* V, const int32_t* kept, const int32_t* sel, int32_t* len, int N, int Hkv,
                          int Lmax, int B, int row_bytes, unsigned long long* rows_moved, hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(N * Hkv * 2), dim3(kCompactThreads), 0, st, (unsigned char*)K, (unsigned char*)V, kept,
                     sel, len, Hkv, Lmax, B, row_bytes, rows_moved);
  return hipGetLastError();
}

}  // namespace bkv

// select.hip -- top-B_KV selection with an always-kept window, and in-place
// compaction of K and V (order-preserving, or hole-filling with positions),
// on gfx950.
//
// Selection (inkeast.github.io MessageDaily paper-reading post on BeaconKV,
// section 三: I = TopK(score(K,V), B_KV); aimodeling.com "BeaconKV: Beacon
// Queries Fix KV Eviction for Long Reasoning", section "Beacon queries
// anticipate what will be revisited": the newest W entries are kept whatever
// their scores).  B_KV counts the window; the other B_KV - W entries are the highest
// scores of the rest, ties at the cut going to the lower index (the older
// position in the hole-filling layout).
//
// select_kernel / select_fill_kernel: one workgroup per (slot, KV head).
// Scores are non-negative floats, so their bit patterns order like the
// values; MSB-first radix selections (4 passes of 8 bits, LDS histograms)
// find each cut value and how many entries equal to it are taken.  A final
// pass gives every thread a contiguous run of entries, so one block scan
// ranks all kept (or evicted) entries in index order.
//
// compact_unit_kernel: row i <- row kept[i] for i from the first evicted
// index up to the kept count, one 1024-thread workgroup per (slot, KV head,
// tensor) walking its rows in 128 KB steps (see its description).  Because
// kept is ascending, kept[i] >= i: a row is only ever read by a destination
// at or before its own index.  compact_kernel: the same walk with 256
// threads and plain global loads, for units whose rows span 2 GB or more
// (beyond the 32-bit offsets of the buffer instructions).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <climits>

#include "bkv_device.hpp"

namespace bkv {

constexpr int kSelThreads = 256;
// Units of at most kStageMax entries read their scores (and positions) once
// into LDS; longer ones read them from global memory on every pass.
constexpr int kStageMax = 4096;

// Copies n 32-bit words to LDS (16-byte loads where aligned); the caller
// synchronises.
__device__ inline void stage_words(uint32_t* dst, const uint32_t* src, int n) {
  const int tid = threadIdx.x;
  if ((((uintptr_t)src) & 15) == 0) {
    const int n4 = n >> 2;
    for (int i = tid; i < n4; i += kSelThreads)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
    for (int i = 4 * n4 + tid; i < n; i += kSelThreads) dst[i] = src[i];
  } else {
    for (int i = tid; i < n; i += kSelThreads) dst[i] = src[i];
  }
}

// hist[b] += 1 for every lane with `active`.  The radix digits of one wave
// are often all equal (scores share their exponent, positions their high
// bytes), and same-address LDS atomics serialise, so lanes holding the most
// common digits are first combined into one atomic each (a few ballot
// rounds); the remaining lanes add individually.  Every lane of the wave must
// call it.
__device__ inline void hist_add(int* hist, uint32_t b, bool active) {
  const int lane = threadIdx.x & 63;
  uint64_t pending = __ballot(active);
#pragma unroll
  for (int round = 0; round < 3; ++round) {
    if (pending == 0) break;
    const int leader = __ffsll((long long)pending) - 1;
    const uint32_t lb = __shfl(b, leader, 64);
    const uint64_t same = __ballot(active && b == lb) & pending;
    if (lane == leader) atomicAdd(&hist[lb], __popcll(same));
    if ((same >> lane) & 1) active = false;
    pending &= ~same;
  }
  if (active) atomicAdd(&hist[b], 1);
}

// Largest-first radix cut over the entries j in [0, n) for which key(j, k)
// returns true (and sets their key k).  Finds the want-th largest key, for
// 1 <= want <= the number of such entries; *take receives how many entries
// equal to it the first `want` include, *n_eq how many entries equal it.
// Every thread of the block must call it with the same arguments.
template <class KeyFn>
__device__ inline uint32_t radix_cut(KeyFn key, int n, int want, int* hist, int* scan_tmp, int* bcast, int* take,
                                     int* n_eq) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  int remaining = want, eq = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int b = tid; b < 256; b += kSelThreads) hist[b] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < n; j0 += kSelThreads) {
      const int j = j0 + tid;
      uint32_t k = 0;
      const bool act = j < n && key(j, k) && (k & mask) == prefix;
      hist_add(hist, (k >> shift) & 255, act);
    }
    __syncthreads();
    const int b = 255 - tid;  // thread t owns bucket 255 - t (kSelThreads == 256)
    const int cnt = hist[b];
    int total;
    const int above = block_exclusive_scan(cnt, scan_tmp, &total);
    if (above < remaining && remaining <= above + cnt) {
      bcast[0] = b;
      bcast[1] = remaining - above;
      bcast[2] = cnt;
    }
    __syncthreads();
    prefix |= (uint32_t)bcast[0] << shift;
    mask |= 255u << shift;
    remaining = bcast[1];
    eq = bcast[2];
    __syncthreads();
  }
  *take = remaining;
  *n_eq = eq;
  return prefix;
}

// Thread t's contiguous run [*a, *b) of [lo, hi).  The run length is odd, so
// the lanes of a wave reading the k-th entry of their runs from LDS hit
// distinct banks.
__device__ inline void thread_run(int lo, int hi, int* a, int* b) {
  const int per = ((hi - lo + kSelThreads - 1) / kSelThreads) | 1;
  *a = min(hi, lo + (int)threadIdx.x * per);
  *b = min(hi, *a + per);
}

// Index of the last of the first `take` entries of [lo, hi) with pred(j),
// in index order (take >= 1 and at most their number).
template <class Pred>
__device__ inline int nth_in_order(int lo, int hi, int take, Pred pred, int* scan_tmp, int* slot) {
  int a, b;
  thread_run(lo, hi, &a, &b);
  int cnt = 0;
  for (int j = a; j < b; ++j) cnt += pred(j) ? 1 : 0;
  int total;
  int r = block_exclusive_scan(cnt, scan_tmp, &total);
  for (int j = a; j < b; ++j)
    if (pred(j)) {
      if (r == take - 1) *slot = j;
      ++r;
    }
  __syncthreads();
  const int v = *slot;
  __syncthreads();
  return v;
}

// Block minimum of one unsigned int per thread.
__device__ inline uint32_t block_min_u32(uint32_t v, int* scan_tmp) {
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = o < v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) scan_tmp[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t m = (uint32_t)scan_tmp[0];
  for (int w = 1; w < kSelThreads / 64; ++w) m = (uint32_t)scan_tmp[w] < m ? (uint32_t)scan_tmp[w] : m;
  __syncthreads();
  return m;
}

// Block minimum of one int per thread.
__device__ inline int block_min(int v, int* scan_tmp) {
  for (int off = 32; off > 0; off >>= 1) {
    const int o = __shfl_xor(v, off, 64);
    v = o < v ? o : v;
  }
  if ((threadIdx.x & 63) == 0) scan_tmp[threadIdx.x >> 6] = v;
  __syncthreads();
  int m = scan_tmp[0];
  for (int w = 1; w < kSelThreads / 64; ++w) m = scan_tmp[w] < m ? scan_tmp[w] : m;
  __syncthreads();
  return m;
}

template <bool kStaged>
__global__ __launch_bounds__(kSelThreads) void select_kernel(const float* __restrict__ scores,
                                                             const int32_t* __restrict__ len, int Hkv, int Lmax,
                                                             int B, int W, int32_t* __restrict__ kept,
                                                             int32_t* __restrict__ sel,
                                                             int32_t* __restrict__ ws_words) {
  static_assert(kSelThreads == 256, "one radix bucket per thread");
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
  extern __shared__ uint32_t stage[];
  const uint32_t* u = reinterpret_cast<const uint32_t*>(scores + unit * (size_t)Lmax);
  if constexpr (kStaged) {
    stage_words(stage, u, L);
    __syncthreads();
    u = stage;
  }
  const int ncand = L - W;  // candidates [0, L - W)
  const int want = B - W;   // how many candidates survive

  // the cut value among the candidates; when entries equal to it straddle
  // the cut, the lowest indices of them are kept up to eq_last
  uint32_t tau = 0;
  int eq_last = 0x7fffffff;
  if (want > 0) {
    int take, neq;
    tau = radix_cut([&](int j, uint32_t& k) { k = u[j]; return true; }, ncand, want, hist, scan_tmp, bcast, &take,
                    &neq);
    if (take < neq) eq_last = nth_in_order(0, ncand, take, [&](int j) { return u[j] == tau; }, scan_tmp, &bcast[3]);
  }
  auto keep = [&](int j) -> bool {
    if (j >= ncand) return true;  // the window
    if (want <= 0) return false;
    const uint32_t x = u[j];
    return x > tau || (x == tau && j <= eq_last);
  };

  // kept indices ascending, and the first evicted index
  int a, b;
  thread_run(0, L, &a, &b);
  int cnt = 0, hole = 0x7fffffff;
  for (int j = a; j < b; ++j) {
    if (keep(j)) ++cnt;
    else if (j < hole) hole = j;
  }
  int total;
  int r = block_exclusive_scan(cnt, scan_tmp, &total);
  for (int j = a; j < b; ++j)
    if (keep(j)) kept_u[r++] = j;
  const int first_hole = block_min(hole, scan_tmp);
  if (tid == 0) {
    sel[2 * unit] = first_hole < B ? first_hole : B;
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

// One workgroup per (slot, KV head, tensor), for units whose rows span 2 GB
// or more (compact_unit_kernel below covers the others).  A step moves
// kCompactUnroll groups of (256 / lanes per row) rows: every thread first waits for its own
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

// ---------------------------------------------------------------------------
// Order-preserving compaction, one workgroup per (unit, tensor)
// ---------------------------------------------------------------------------
//
// A step moves the destinations [i0, i0 + SR): every lane loads kUnitLoads
// 16-byte pieces (rows i0 + r0 + b * RPP, b < kUnitLoads), so a step is
// kUnitThreads * kUnitLoads * 16 bytes.  Its loads read rows kept[i] >= i,
// at or beyond i0, which no earlier step writes; its stores go out after the
// loads of every lane for this and all earlier steps have returned (each
// lane waits for its own loads, then one barrier), and the rows it
// overwrites are read only by destinations at or before them, loaded
// already.  So the next step's loads are issued before this step's stores.
// A store keeps its data registers until it completes, so three register
// sets rotate and a set is loaded again two steps after its stores went out
// (with two sets every step's loads waited for the previous step's stores).
// Rows outside [f, cnt) take an offset past the end of the buffer
// descriptor: such a load returns zero and such a store is dropped, without
// a memory access, so all lanes issue the same instructions.  The kept
// indices are staged in LDS, kUnitWindow at a time.  The window's LDS (just
// over 80 KB) also limits a CU to one such workgroup, as do its registers
// (over 64 per lane at 1024 lanes): 256 (unit, tensor) regions are
// streamed at once, each contiguous, which measured faster than two
// workgroups per CU and than 64 KB chunks of many units in flight together
// (HBM pages are only hit densely when the rows in flight are).

constexpr int kUnitThreads = 1024;
constexpr int kUnitLoads = 8;         // 16-byte loads per lane and step (128 KB steps)
constexpr int kUnitWindow = 20480;    // kept indices staged in LDS at a time
constexpr int kUnitLdsWords = kUnitWindow + 64;  // just over half of a CU's 160 KB of LDS
constexpr int kUnitRsrcWord3 = 0x00020000;  // raw buffer descriptor, word 3 (32-bit data format)
constexpr int kNtAux = 2;             // non-temporal cache policy of the buffer instructions

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int LPR>  // lanes per row: row bytes / 16
__global__ __launch_bounds__(kUnitThreads) void compact_unit_kernel(
    unsigned char* __restrict__ K, unsigned char* __restrict__ V, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ sel, int32_t* __restrict__ len, int Hkv, int Lmax, int B,
    unsigned long long* __restrict__ rows_moved) {
  constexpr int RB = LPR * 16;                 // row bytes
  constexpr int RPP = kUnitThreads / LPR;      // rows between a lane's pieces
  constexpr int SR = RPP * kUnitLoads;         // rows per step
  static_assert(kUnitWindow % SR == 0, "a window holds whole steps");
  __shared__ int s_idx[kUnitLdsWords];
  const size_t unit = blockIdx.x >> 1;
  const int tensor = blockIdx.x & 1;
  const int tid = threadIdx.x;
  const int f = sel[2 * unit];
  const int cnt = sel[2 * unit + 1];
  if (cnt < 0) return;  // unit rejected by the selection
  if (tid == 0) {
    if (tensor == 0 && unit % Hkv == 0) len[unit / Hkv] = cnt;  // no compaction block reads len
    if (cnt > f) atomicAdd(rows_moved, (unsigned long long)(cnt - f));
  }
  if (cnt <= f) return;
  const int32_t* kept_u = kept + unit * (size_t)B;
  const int nrec = Lmax * RB;  // < 2^31 (checked on the host)
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (tensor ? V : K) + unit * (size_t)Lmax * RB, (short)0, nrec, kUnitRsrcWord3);
  const int r0 = tid / LPR;
  const int col = (tid % LPR) * 16;
  for (int w0 = f; w0 < cnt; w0 += kUnitWindow) {
    const int w1 = min(cnt, w0 + kUnitWindow);
    for (int i = w0 + tid; i < w1; i += kUnitThreads) s_idx[i - w0] = kept_u[i];
    __syncthreads();
    auto issue = [&](u32x4* dst, int i0) {
#pragma unroll
      for (int b = 0; b < kUnitLoads; ++b) {
        const int i = i0 + r0 + b * RPP;
        dst[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, i < w1 ? s_idx[i - w0] * RB + col : nrec, 0, kNtAux);
      }
    };
    auto put = [&](const u32x4* src, int i0) {
#pragma unroll
      for (int b = 0; b < kUnitLoads; ++b) {
        const int i = i0 + r0 + b * RPP;
        __builtin_amdgcn_raw_buffer_store_b128(src[b], rs, i < w1 ? i * RB + col : nrec, 0, kNtAux);
      }
    };
    // waits for this lane's loads into x (the compiler counts the stores
    // issued after them, which stay in flight)
    auto landed = [&](const u32x4* x) {
#pragma unroll
      for (int b = 0; b < kUnitLoads; ++b) __asm__ volatile("" ::"v"(x[b]));
    };
    u32x4 a[kUnitLoads], c[kUnitLoads], e[kUnitLoads];
    issue(a, w0);
    landed(a);
    int i0 = w0;
    while (true) {
      __syncthreads();  // every lane's loads of the step at i0 have returned
      if (i0 + SR < w1) issue(c, i0 + SR);
      put(a, i0);
      i0 += SR;
      if (i0 >= w1) break;
      landed(c);
      __syncthreads();
      if (i0 + SR < w1) issue(e, i0 + SR);
      put(c, i0);
      i0 += SR;
      if (i0 >= w1) break;
      landed(e);
      __syncthreads();
      if (i0 + SR < w1) issue(a, i0 + SR);
      put(e, i0);
      i0 += SR;
      if (i0 >= w1) break;
      landed(a);
    }
    __syncthreads();  // the next window's staging overwrites s_idx
  }
}

// ---------------------------------------------------------------------------
// Hole-filling layout
//
// Rows carry their token positions (pos[N][Hkv][Lmax]), so the cache need not
// stay in position order.  select_fill_kernel keeps the W newest positions
// (ties: the lower row) and the B - W highest scores of the other rows (ties:
// the older position, then the lower row).  Each of these orders is found by
// radix cuts over 32-bit keys that order like the quantity; a further cut
// runs only when entries tie at a cut.  The evicted rows of [0, B) ("holes")
// are then paired, in ascending order, with the kept rows of [B, L)
// ("fillers"): kept[i] = i for a kept row below B, else its filler.
// compact_fill_kernel moves only the fillers.  Destinations lie below B and
// sources at or beyond it, so no copy reads a row that another one writes.

constexpr int kFillChunk = 1024;  // fillers paired per sweep (LDS list)
constexpr int kFillBatch = 8;     // 16-byte pieces in flight per thread (named registers below)

// Copies K and V rows src[q] -> dst[q] (q < npairs, lists in LDS) of one unit
// with all 256 threads, kFillBatch 16-byte loads per thread in flight before
// the matching stores.  Sources and destinations must not overlap.
__device__ __forceinline__ void copy_row_pairs(unsigned char* kb, unsigned char* vb, int row_bytes, const int* src,
                                               const int* dst, int npairs) {
  const int tid = threadIdx.x;
  const int lpr = row_bytes / 16;  // 16-byte pieces per row
  const int items = npairs * 2 * lpr;  // (row, tensor, piece)
  // byte offset of piece `it` in the K (tensor 0) or V row of pair `mv`
  auto piece = [&](int it, const int* rows, unsigned char** base) -> size_t {
    const int mv = it / (2 * lpr), rem = it - mv * 2 * lpr;
    *base = rem >= lpr ? vb : kb;
    return (size_t)rows[mv] * row_bytes + (size_t)(rem >= lpr ? rem - lpr : rem) * 16;
  };
  for (int it0 = tid; it0 < items; it0 += 256 * kFillBatch) {
    // past the end the last piece is loaded again and not stored
    unsigned char* b;
#define BKV_FILL_LD(k)                                                                     \
  const int pc##k = min(it0 + (k) * 256, items - 1);                                       \
  const size_t so##k = piece(pc##k, src, &b);                                              \
  const uint4 v##k = *reinterpret_cast<const uint4*>(b + so##k);
#define BKV_FILL_ST(k)                                                                     \
  if (it0 + (k) * 256 < items) {                                                           \
    const size_t d##k = piece(pc##k, dst, &b);                                             \
    *reinterpret_cast<uint4*>(b + d##k) = v##k;                                            \
  }
    BKV_FILL_LD(0) BKV_FILL_LD(1) BKV_FILL_LD(2) BKV_FILL_LD(3)
    BKV_FILL_LD(4) BKV_FILL_LD(5) BKV_FILL_LD(6) BKV_FILL_LD(7)
    BKV_FILL_ST(0) BKV_FILL_ST(1) BKV_FILL_ST(2) BKV_FILL_ST(3)
    BKV_FILL_ST(4) BKV_FILL_ST(5) BKV_FILL_ST(6) BKV_FILL_ST(7)
#undef BKV_FILL_LD
#undef BKV_FILL_ST
  }
}

// kCompact: also moves the filler rows (K, V, positions) into their holes as
// soon as a chunk of pairs is known, leaving nothing for compact_fill_kernel
// (the select table then reads "no hole").  Needs the staged positions (the
// selection keeps reading the old ones while holes are filled); the caller
// updates len afterwards.
template <bool kStaged, bool kCompact>
__global__ __launch_bounds__(kSelThreads) void select_fill_kernel(const float* __restrict__ scores,
                                                                  int32_t* __restrict__ pos,
                                                                  const int32_t* __restrict__ len, int Hkv, int Lmax,
                                                                  int B, int W, int32_t* __restrict__ kept,
                                                                  int32_t* __restrict__ sel,
                                                                  int32_t* __restrict__ ws_words,
                                                                  unsigned char* __restrict__ K,
                                                                  unsigned char* __restrict__ V, int row_bytes,
                                                                  unsigned long long* __restrict__ rows_moved) {
  static_assert(kSelThreads == 256, "one radix bucket per thread");
  static_assert(kStaged || !kCompact, "filling in place needs the staged positions");
  __shared__ int hist[256];
  __shared__ int scan_tmp[16];
  __shared__ int bcast[4];
  __shared__ int fillers[kFillChunk];
  __shared__ int holes[kCompact ? kFillChunk : 1];
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
  extern __shared__ uint32_t stage[];
  const uint32_t* u = reinterpret_cast<const uint32_t*>(scores + unit * (size_t)Lmax);
  const int32_t* pp = pos + unit * (size_t)Lmax;
  if constexpr (kStaged) {
    stage_words(stage, u, L);
    const int ls = (Lmax + 3) & ~3;  // positions follow the scores, 16-byte aligned
    stage_words(stage + ls, reinterpret_cast<const uint32_t*>(pp), L);
    __syncthreads();
    u = stage;
    pp = reinterpret_cast<const int32_t*>(stage + ls);
  }
  // signed positions -> unsigned keys in the same order
  auto pkey = [pp](int j) { return (uint32_t)pp[j] ^ 0x80000000u; };

  // the window: the W largest position keys, ties to the lower row.  When the
  // last W rows hold positions above every other row's (tokens appended in
  // order since the last eviction), they are that window; otherwise radix
  // cuts find it.
  uint32_t wt = 0;
  int wrow = 0x7fffffff;
  bool tail_window = false;
  if (W > 0) {
    uint32_t head_max = 0u, tail_min = 0xFFFFFFFFu;
    for (int j = tid; j < L; j += kSelThreads) {
      const uint32_t k = pkey(j);
      if (j < L - W) head_max = k > head_max ? k : head_max;
      else tail_min = k < tail_min ? k : tail_min;
    }
    head_max = ~block_min_u32(~head_max, scan_tmp);  // max(x) = ~min(~x)
    tail_min = block_min_u32(tail_min, scan_tmp);
    tail_window = tail_min > head_max;
  }
  if (W > 0 && !tail_window) {
    int take, neq;
    wt = radix_cut([&](int j, uint32_t& k) { k = pkey(j); return true; }, L, W, hist, scan_tmp, bcast, &take, &neq);
    if (take < neq)  // equal positions straddle the cut: the lowest rows of them
      wrow = nth_in_order(0, L, take, [&](int j) { return pkey(j) == wt; }, scan_tmp, &bcast[3]);
  }
  auto in_win = [&](int j) -> bool {
    if (W == 0) return false;
    if (tail_window) return j >= L - W;
    const uint32_t k = pkey(j);
    return k > wt || (k == wt && j <= wrow);
  };

  // the others: B - W highest scores, ties to the older position, then the lower row
  const int want = B - W;
  uint32_t st = 0, pt = 0;
  bool all_st = true, all_pt = true;
  int prow = 0x7fffffff;
  if (want > 0) {
    int take, neq;
    st = radix_cut([&](int j, uint32_t& k) { k = u[j]; return !in_win(j); }, L, want, hist, scan_tmp, bcast, &take,
                   &neq);
    if (take < neq) {
      all_st = false;
      int t2, n2;
      pt = radix_cut([&](int j, uint32_t& k) { k = ~pkey(j); return u[j] == st && !in_win(j); }, L, take, hist,
                     scan_tmp, bcast, &t2, &n2);
      if (t2 < n2) {
        all_pt = false;
        prow = nth_in_order(0, L, t2, [&](int j) { return u[j] == st && ~pkey(j) == pt && !in_win(j); }, scan_tmp,
                            &bcast[3]);
      }
    }
  }
  auto keep = [&](int j) -> bool {
    if (in_win(j)) return true;
    if (want <= 0) return false;
    const uint32_t x = u[j];
    if (x != st) return x > st;
    if (all_st) return true;
    const uint32_t k2 = ~pkey(j);
    if (k2 != pt) return k2 > pt;
    return all_pt || j <= prow;
  };

  // pair the holes of [0, B) with the fillers of [B, L), kFillChunk at a
  // time (one predicate evaluation per row and sweep: cheaper here than
  // contiguous runs, which evaluate each row three times)
  int hole = 0x7fffffff;
  for (int r0 = 0;; r0 += kFillChunk) {
    int base = 0;
    for (int j0 = B; j0 < L; j0 += kSelThreads) {
      const int j = j0 + tid;
      const bool f = j < L && keep(j);
      int tot;
      const int r = base + block_exclusive_scan(f ? 1 : 0, scan_tmp, &tot);
      if (f && r >= r0 && r < r0 + kFillChunk) fillers[r - r0] = j;
      base += tot;
    }
    const int nfill = base;
    __syncthreads();
    int hbase = 0;
    for (int i0 = 0; i0 < B; i0 += kSelThreads) {
      const int i = i0 + tid;
      const bool h = i < B && !keep(i);
      int tot;
      const int r = hbase + block_exclusive_scan(h ? 1 : 0, scan_tmp, &tot);
      if (i < B) {
        if (!h) {
          if (r0 == 0) kept_u[i] = i;
        } else {
          if (i < hole) hole = i;
          // r < nfill always (as many holes as fillers); the guard keeps every
          // LDS read inside the filled part of the list
          if (r >= r0 && r < r0 + kFillChunk) {
            kept_u[i] = r < nfill ? fillers[r - r0] : i;
            if constexpr (kCompact) {
              if (r < nfill) holes[r - r0] = i;  // every rank below nfill has one hole
            }
          }
        }
      }
      hbase += tot;
    }
    __syncthreads();
    if constexpr (kCompact) {
      // this chunk's pairs: rows and positions (the selection reads the staged copies)
      const int np = min(kFillChunk, nfill - r0);
      const size_t ub = unit * (size_t)Lmax;
      copy_row_pairs(K + ub * row_bytes, V + ub * row_bytes, row_bytes, fillers, holes, np);
      for (int q = tid; q < np; q += kSelThreads) pos[ub + holes[q]] = pp[fillers[q]];
      if (tid == 0 && np > 0) atomicAdd(rows_moved, 2ull * (unsigned long long)np);  // K and V rows
      __syncthreads();  // the lists are rewritten by the next sweep
    }
    if (r0 + kFillChunk >= nfill) break;
  }
  const int first_hole = block_min(hole, scan_tmp);
  if (tid == 0) {
    sel[2 * unit] = kCompact ? B : (first_hole < B ? first_hole : B);
    sel[2 * unit + 1] = B;
  }
}

// len[n] <- min(len[n], B) for valid lengths (after the fused selection and fill).
__global__ void fill_len_kernel(int32_t* __restrict__ len, int N, int Lmax, int B) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) {
    const int L = len[n];
    if (L > B && L <= Lmax) len[n] = B;
  }
}

// One workgroup per (slot, KV head): K, V and the positions.  Rows from the
// first hole to the kept count are scanned kCompactThreads at a time; the
// rows whose gather index differs from their own are listed in LDS and their
// K and V pieces copied in batches of kFillBatch loads per thread before the
// matching stores.
__global__ __launch_bounds__(kCompactThreads) void compact_fill_kernel(unsigned char* __restrict__ K,
                                                                       unsigned char* __restrict__ V,
                                                                       int32_t* __restrict__ pos,
                                                                       const int32_t* __restrict__ kept,
                                                                       int32_t* __restrict__ sel,
                                                                       int32_t* __restrict__ len, int Hkv, int Lmax,
                                                                       int B, int row_bytes,
                                                                       unsigned long long* __restrict__ rows_moved) {
  __shared__ int mv_dst[kCompactThreads];
  __shared__ int mv_src[kCompactThreads];
  __shared__ int scan_tmp[16];
  const size_t unit = blockIdx.x;
  const int tid = threadIdx.x;
  const int f = sel[2 * unit];
  const int cnt = sel[2 * unit + 1];
  if (cnt < 0) return;  // unit rejected by the selection
  const int n = (int)(unit / Hkv);
  if (tid == 0 && unit % Hkv == 0) len[n] = cnt;  // no compaction block reads len
  if (cnt <= f) return;
  const int32_t* kept_u = kept + unit * (size_t)B;
  unsigned char* kb = K + unit * (size_t)Lmax * row_bytes;
  unsigned char* vb = V + unit * (size_t)Lmax * row_bytes;
  int32_t* pu = pos + unit * (size_t)Lmax;
  int moved = 0;
  for (int i0 = f; i0 < cnt; i0 += kCompactThreads) {
    const int i = i0 + tid;
    const int src = i < cnt ? kept_u[i] : i;
    // fillers lie at or beyond the kept count (and inside the allocation)
    const bool m = src != i && src >= cnt && src < Lmax;
    int nm;
    const int r = block_exclusive_scan(m ? 1 : 0, scan_tmp, &nm);
    if (m) {
      mv_dst[r] = i;
      mv_src[r] = src;
    }
    __syncthreads();
    copy_row_pairs(kb, vb, row_bytes, mv_src, mv_dst, nm);
    if (tid < nm) pu[mv_dst[tid]] = pu[mv_src[tid]];
    moved += nm;
    __syncthreads();  // the lists are rewritten by the next sweep
  }
  if (tid == 0) {
    if (moved > 0) atomicAdd(rows_moved, 2ull * (unsigned long long)moved);  // K and V rows
    sel[2 * unit] = cnt;  // no hole left: a repeated call moves nothing
  }
}

hipError_t launch_select(const float* scores, const int32_t* len, int N, int Hkv, int Lmax, int B, int W,
                         int32_t* kept, int32_t* sel, int32_t* ws_words, hipStream_t st) {
  if (Lmax <= kStageMax)
    hipLaunchKernelGGL(select_kernel<true>, dim3(N * Hkv), dim3(kSelThreads), Lmax * sizeof(uint32_t), st, scores,
                       len, Hkv, Lmax, B, W, kept, sel, ws_words);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3(N * Hkv), dim3(kSelThreads), 0, st, scores, len, Hkv, Lmax, B, W,
                       kept, sel, ws_words);
  return hipGetLastError();
}

// The order-preserving compaction: one block per (unit, tensor); the
// 1024-thread kernel where a unit's rows span less than 2 GB, else the
// 256-thread one with 64-bit addresses.  Needs no workspace beyond the select
// table.
hipError_t launch_compact(void* K, void* V, const int32_t* kept, const int32_t* sel, int32_t* len, int N, int Hkv,
                          int Lmax, int B, int row_bytes, unsigned long long* rows_moved, hipStream_t st) {
  const size_t units = (size_t)N * Hkv;
  if (units == 0) return hipSuccess;
  const dim3 grid((unsigned)(2 * units));
  unsigned char* k = (unsigned char*)K;
  unsigned char* v = (unsigned char*)V;
  if ((size_t)Lmax * row_bytes <= (size_t)INT32_MAX) {
    switch (row_bytes) {
      case 128:
        hipLaunchKernelGGL(compact_unit_kernel<8>, grid, dim3(kUnitThreads), 0, st, k, v, kept, sel, len, Hkv, Lmax,
                           B, rows_moved);
        return hipGetLastError();
      case 256:
        hipLaunchKernelGGL(compact_unit_kernel<16>, grid, dim3(kUnitThreads), 0, st, k, v, kept, sel, len, Hkv, Lmax,
                           B, rows_moved);
        return hipGetLastError();
      case 512:
        hipLaunchKernelGGL(compact_unit_kernel<32>, grid, dim3(kUnitThreads), 0, st, k, v, kept, sel, len, Hkv, Lmax,
                           B, rows_moved);
        return hipGetLastError();
      default:
        break;
    }
  }
  hipLaunchKernelGGL(compact_kernel, grid, dim3(kCompactThreads), 0, st, k, v, kept, sel, len, Hkv, Lmax, B, row_bytes,
                     rows_moved);
  return hipGetLastError();
}

hipError_t launch_select_fill(const float* scores, const int32_t* pos, const int32_t* len, int N, int Hkv, int Lmax,
                              int B, int W, int32_t* kept, int32_t* sel, int32_t* ws_words, hipStream_t st) {
  int32_t* p = const_cast<int32_t*>(pos);  // read only without kCompact
  if (Lmax <= kStageMax)
    hipLaunchKernelGGL((select_fill_kernel<true, false>), dim3(N * Hkv), dim3(kSelThreads),
                       2 * ((Lmax + 3) & ~3) * sizeof(uint32_t), st, scores, p, len, Hkv, Lmax, B, W, kept, sel,
                       ws_words, nullptr, nullptr, 0, nullptr);
  else
    hipLaunchKernelGGL((select_fill_kernel<false, false>), dim3(N * Hkv), dim3(kSelThreads), 0, st, scores, p, len,
                       Hkv, Lmax, B, W, kept, sel, ws_words, nullptr, nullptr, 0, nullptr);
  return hipGetLastError();
}

// Selection and hole filling in one kernel where the unit is staged in LDS,
// else the two kernels.
hipError_t launch_select_compact_fill(const float* scores, void* K, void* V, int32_t* pos, int32_t* len, int N,
                                      int Hkv, int Lmax, int B, int W, int32_t* kept, int32_t* sel, int row_bytes,
                                      unsigned long long* rows_moved, int32_t* ws_words, hipStream_t st);

hipError_t launch_compact_fill(void* K, void* V, int32_t* pos, const int32_t* kept, int32_t* sel, int32_t* len,
                               int N, int Hkv, int Lmax, int B, int row_bytes, unsigned long long* rows_moved,
                               hipStream_t st) {
  hipLaunchKernelGGL(compact_fill_kernel, dim3(N * Hkv), dim3(kCompactThreads), 0, st, (unsigned char*)K,
                     (unsigned char*)V, pos, kept, sel, len, Hkv, Lmax, B, row_bytes, rows_moved);
  return hipGetLastError();
}

hipError_t launch_select_compact_fill(const float* scores, void* K, void* V, int32_t* pos, int32_t* len, int N,
                                      int Hkv, int Lmax, int B, int W, int32_t* kept, int32_t* sel, int row_bytes,
                                      unsigned long long* rows_moved, int32_t* ws_words, hipStream_t st) {
  if (Lmax > kStageMax) {
    hipError_t e = launch_select_fill(scores, pos, len, N, Hkv, Lmax, B, W, kept, sel, ws_words, st);
    if (e != hipSuccess) return e;
    return launch_compact_fill(K, V, pos, kept, sel, len, N, Hkv, Lmax, B, row_bytes, rows_moved, st);
  }
  hipLaunchKernelGGL((select_fill_kernel<true, true>), dim3(N * Hkv), dim3(kSelThreads),
                     2 * ((Lmax + 3) & ~3) * sizeof(uint32_t), st, scores, pos, len, Hkv, Lmax, B, W, kept, sel,
                     ws_words, (unsigned char*)K, (unsigned char*)V, row_bytes, rows_moved);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fill_len_kernel, dim3((N + 255) / 256), dim3(256), 0, st, len, N, Lmax, B);
  return hipGetLastError();
}

}  // namespace bkv

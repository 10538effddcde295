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
// compact_chunk_kernel: row i <- row kept[i] for i from the first evicted
// index up to the kept count, in chunks of 64 KB of rows, one workgroup each
// (see its description).  Because kept is ascending, kept[i] >= i: a
// row is only ever read by a destination at or before its own index.
// compact_kernel: the same move with one workgroup per (slot, KV head,
// tensor), in steps of increasing index; a block-wide barrier after each
// step's loads have returned orders every read of a row before its
// overwrite.  It needs no workspace beyond the select table.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

// ---------------------------------------------------------------------------
// Chunked order-preserving compaction
// ---------------------------------------------------------------------------
//
// The rows of a (unit, tensor) are cut into chunks of CR = kChunkBytes /
// row_bytes rows, one workgroup each; chunk j moves the destinations [s_j,
// e_j) = [j CR, (j + 1) CR) within [f, cnt) (f the first hole, cnt the kept
// count).  It reads kept[i] >= i for i in [s_j, e_j): a later chunk reads
// only rows at or beyond its own first destination, above every row chunk j
// writes, and chunk j's own reads all return before its first store.  The
// one hazard left is a row chunk j overwrites that an earlier chunk j' still
// reads: a source of j' at or beyond s_j, which exists only while the last
// source of j', kept[e_j' - 1], is >= s_j (at most (L - cnt) / CR + 1
// earlier chunks).  So each chunk loads all its rows into registers,
// publishes "read" in its flag, waits for the flags of the earlier chunks that
// reach into its rows, then stores.  Blocks are numbered chunk-major, so an
// earlier chunk of the same (unit, tensor) has a lower block index: each XCD
// dispatches its blocks in index order, so while a block waits every
// lower-indexed block is running or done, and it publishes its flag before
// waiting on anything; the wait is also bounded (BKV_DEV_WAIT_LIMIT).  A
// block has no stores outstanding when it waits for its loads, so its flag
// follows its reads alone.  compact_prepare_kernel clears the flags before
// every call (a kernel, not a memset node, so that the call can be captured
// into a graph).

constexpr int kChunkBytes = 65536;                                    // bytes of rows per chunk
constexpr int kChunkPieces = kChunkBytes / 16 / kCompactThreads;     // 16-byte loads per thread
constexpr int kChunkWaitPolls = 1 << 22;                              // bound of one flag wait (seconds)

__host__ __device__ inline int compact_chunk_rows(int row_bytes) { return kChunkBytes / row_bytes; }

// Zeroes the chunk flags.
__global__ void compact_prepare_kernel(uint32_t* flags, size_t words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += (size_t)gridDim.x * blockDim.x)
    flags[i] = 0u;
}

__global__ __launch_bounds__(kCompactThreads) void compact_chunk_kernel(
    unsigned char* __restrict__ K, unsigned char* __restrict__ V, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ sel, int32_t* __restrict__ len, int Hkv, int Lmax, int B, int row_bytes,
    unsigned long long* __restrict__ rows_moved, uint32_t* __restrict__ flags, int units, int nchunk,
    int32_t* __restrict__ ws_words) {
  __shared__ int s_go;
  const int tid = threadIdx.x;
  const uint32_t items_per_chunk = 2u * (uint32_t)units;
  const int j = (int)(blockIdx.x / items_per_chunk);
  const uint32_t ut = blockIdx.x % items_per_chunk;  // (unit, tensor)
  const size_t unit = ut >> 1;
  const int tensor = (int)(ut & 1u);
  const int lpr = row_bytes / 16;
  const int CR = compact_chunk_rows(row_bytes);
  const int c0 = j * CR;  // chunk j: destinations [c0, c0 + CR) within [f, cnt)
  const int32_t* kept_u = kept + unit * (size_t)B;
  // the kept indices of the chunk's rows go out with the select table entry
  // (kept[i] = i below the first hole, so reading them needs no f)
  const int rows_here = max(0, min(CR, B - c0));
  int src[kChunkPieces];
#pragma unroll
  for (int b = 0; b < kChunkPieces; ++b) {
    const int r = (b * kCompactThreads + tid) / lpr;
    src[b] = r < rows_here ? kept_u[c0 + r] : 0;
  }
  const int f = sel[2 * unit];
  const int cnt = sel[2 * unit + 1];
  if (cnt < 0) return;  // unit rejected by the selection
  if (j == 0 && tid == 0) {
    if (tensor == 0 && unit % Hkv == 0) len[unit / Hkv] = cnt;  // no compaction block reads len
    if (cnt > f) atomicAdd(rows_moved, (unsigned long long)(cnt - f));
  }
  const int start = max(f, c0);
  const int end = min(cnt, c0 + CR);
  if (start >= end) return;  // nothing of this chunk moves
  uint32_t* uflags = flags + ut * (size_t)nchunk;
  // the nearest earlier chunk, if it moves rows and its reads reach into this
  // chunk's rows (its flag is read alongside the rows; usually set long since)
  const bool dep = j > 0 && c0 - 1 >= f && kept_u[c0 - 1] >= start;
  uint32_t early = 1u;
  if (tid == 0 && dep) early = __hip_atomic_load(&uflags[j - 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  unsigned char* base = (tensor ? V : K) + unit * (size_t)Lmax * row_bytes;
  nt_u32x4 v[kChunkPieces];
#pragma unroll
  for (int b = 0; b < kChunkPieces; ++b) {
    const int p = b * kCompactThreads + tid;
    const int r = p / lpr;
    if (c0 + r >= start && c0 + r < end) v[b] = nt_load16(base + (size_t)src[b] * row_bytes + (size_t)(p - r * lpr) * 16);
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();  // every row of the chunk has been read
  if (tid == 0) {
    __hip_atomic_store(&uflags[j], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int go = 1;
    if (dep) {
      // the earlier chunks that move rows and whose last source lies at or
      // beyond this chunk's first moved row: the nearest one (read above),
      // then further back
      for (int jp = j - 1; jp >= 0 && go; --jp) {
        const int last = (jp + 1) * CR - 1;  // last destination of chunk jp (jp < j: a whole chunk)
        if (last < f || kept_u[last] < start) break;
        uint32_t fl = jp == j - 1 ? early : 0u;
        for (int polls = 0; fl == 0u; ++polls) {
          if (polls >= kChunkWaitPolls) {
            go = 0;
            set_status(ws_words, BKV_DEV_WAIT_LIMIT);
            break;
          }
          if (polls > 0) __builtin_amdgcn_s_sleep(2);
          fl = __hip_atomic_load(&uflags[jp], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
    }
    s_go = go;
  }
  __syncthreads();
  if (!s_go) return;  // a wait passed its bound: this chunk's rows are left unwritten
#pragma unroll
  for (int b = 0; b < kChunkPieces; ++b) {
    const int p = b * kCompactThreads + tid;
    const int r = p / lpr;
    if (c0 + r >= start && c0 + r < end) nt_store16(base + (size_t)(c0 + r) * row_bytes + (size_t)(p - r * lpr) * 16, v[b]);
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

// One block per (unit, tensor), stepping through its rows (no workspace
// beyond the select table).
hipError_t launch_compact_stepped(void* K, void* V, const int32_t* kept, const int32_t* sel, int32_t* len, int N,
                                  int Hkv, int Lmax, int B, int row_bytes, unsigned long long* rows_moved,
                                  hipStream_t st) {
  hipLaunchKernelGGL(compact_kernel, dim3(N * Hkv * 2), dim3(kCompactThreads), 0, st, (unsigned char*)K, (unsigned char*)V, kept,
                     sel, len, Hkv, Lmax, B, row_bytes, rows_moved);
  return hipGetLastError();
}

// Words of the chunked compaction's flags.
size_t compact_area_words(int units, int Lmax, int row_bytes) {
  const int cr = compact_chunk_rows(row_bytes);
  const size_t nchunk = Lmax > 0 ? ((size_t)Lmax + cr - 1) / cr : 1;
  return 2 * (size_t)units * nchunk;
}

// The chunked compaction: the flags cleared, then one block per (chunk, unit,
// tensor), chunk-major.
hipError_t launch_compact(void* K, void* V, const int32_t* kept, const int32_t* sel, int32_t* len, int N, int Hkv,
                          int Lmax, int B, int row_bytes, unsigned long long* rows_moved, uint32_t* flags,
                          int32_t* ws_words, hipStream_t st) {
  const int units = N * Hkv;
  if (units == 0) return hipSuccess;
  const int cr = compact_chunk_rows(row_bytes);
  const int nchunk = Lmax > 0 ? (Lmax + cr - 1) / cr : 1;
  const size_t words = compact_area_words(units, Lmax, row_bytes);
  hipLaunchKernelGGL(compact_prepare_kernel, dim3((unsigned)std::min<size_t>((words + 255) / 256, 1024)), dim3(256), 0,
                     st, flags, words);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(compact_chunk_kernel, dim3((unsigned)(2 * (size_t)units * nchunk)), dim3(kCompactThreads), 0, st,
                     (unsigned char*)K, (unsigned char*)V, kept, sel, len, Hkv, Lmax, B, row_bytes, rows_moved, flags,
                     units, nchunk, ws_words);
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

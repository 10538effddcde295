// bkv_api.hip -- host side of the libbkv C ABI (argument checks, workspace
// layout, kernel dispatch).  Declarations and contracts: include/bkv.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <stdint.h>

#include <mutex>

#include "bkv.h"
#include "bkv_device.hpp"

namespace bkv {

template <int DT, int D>
hipError_t launch_fps_update(const void*, int, void*, int32_t*, int, int, int, int32_t*, hipStream_t);
template <int DT, int D>
hipError_t launch_beacon_picks(const void*, const int32_t*, int, int, int, int32_t*, void*, int32_t*, hipStream_t);
template <int DT, int D>
hipError_t launch_score(const void*, const int32_t*, int, int, int, int, const void*, const int32_t*, int,
                        const int32_t*, const void*, int, const int32_t*, double, float2*, void*, int32_t*, int,
                        float*, float*, int32_t*, bool, const float*, hipStream_t);
template <int DT, int D>
hipError_t launch_decode(const void*, const void*, const void*, const int32_t*, int, int, int, int, float*, float*,
                         float*, int32_t*, hipStream_t);
hipError_t launch_beacon_rows(const void*, int, const int32_t*, int, int, int, int32_t*, void*, int32_t*,
                              hipStream_t);
hipError_t launch_select(const float*, const int32_t*, int, int, int, int, int, int32_t*, int32_t*, int32_t*,
                         hipStream_t);
hipError_t launch_compact(void*, void*, const int32_t*, const int32_t*, int32_t*, int, int, int, int, int,
                          unsigned long long*, hipStream_t);
hipError_t launch_select_fill(const float*, const int32_t*, const int32_t*, int, int, int, int, int, int32_t*,
                              int32_t*, int32_t*, hipStream_t);
hipError_t launch_compact_fill(void*, void*, int32_t*, const int32_t*, int32_t*, int32_t*, int, int, int, int, int,
                               unsigned long long*, hipStream_t);
hipError_t launch_select_compact_fill(const float*, void*, void*, int32_t*, int32_t*, int, int, int, int, int,
                                      int32_t*, int32_t*, int, unsigned long long*, int32_t*, hipStream_t);

template <int DT, int D>
hipError_t launch_fps_full(const void*, long, long, int, int32_t*, void*, hipStream_t);
size_t fps_full_workspace_bytes(long, long, int);

__global__ void zero_header_kernel(int32_t* w) {
  if (threadIdx.x < (int)(kHeaderBytes / 4)) w[threadIdx.x] = 0;
}

__global__ void copy_status_kernel(const int32_t* __restrict__ w, int32_t* __restrict__ out) {
  if (threadIdx.x == 0) out[0] = w[kStatusWord];
}

// Scratch memory of bkv_select_compact_noalloc: the workspace header (status
// word, rows_moved) followed by the select table [N][Hkv][2].  Each device
// holds its own copy, at its own address, for the life of the process.
constexpr size_t kNoallocScratchBytes = size_t(1) << 20;
constexpr long kNoallocMaxUnits = (long)((kNoallocScratchBytes - kHeaderBytes) / (2 * sizeof(int32_t)));
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device, once looked up

// The device address of the current device's `scratch` (looked up on the
// first call on that device; the host-side name of the array is not a
// device address and is never passed to a kernel).
int scratch_on_current_device(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return BKV_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return BKV_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = (unsigned char*)g_scratch_ptr[dev];
  return BKV_OK;
}

}  // namespace

namespace {

constexpr int kMaxCapacity = 256;
constexpr int kMaxRows = 256;
constexpr int kMaxRecent = 64;
constexpr int kMaxLen = 1 << 24;
constexpr int kMaxHistory = 1 << 24;
constexpr int kMaxFullPicks = 4096;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int elem_bytes(int dtype) { return dtype == BKV_F32 ? 4 : 2; }

int check_shape(const bkv_shape* s) {
  if (!s) return BKV_E_NULL;
  if (s->dtype != BKV_F32 && s->dtype != BKV_BF16) return BKV_E_DTYPE;
  if (s->n_seq < 0 || s->n_kv_heads < 1 || s->n_q_heads < s->n_kv_heads || s->n_q_heads % s->n_kv_heads != 0)
    return BKV_E_SHAPE;
  if (s->head_dim != 64 && s->head_dim != 128) return BKV_E_SHAPE;
  if (s->max_len < 0 || s->max_len > kMaxLen) return BKV_E_SHAPE;
  return BKV_OK;
}

struct WsLayout {
  size_t obs, valid, lse, select, rope, beacons, beacon_rows, total;
  int RP;
};

// Header, then the select table (it depends on the shape only, so
// bkv_select and bkv_compact need no R or nb), then the scoring
// intermediates.
size_t select_end(const bkv_shape* s) {
  return align256(kHeaderBytes + (size_t)s->n_seq * s->n_kv_heads * 2 * sizeof(int32_t));
}

bool layout(const bkv_shape* s, int R, int nb, WsLayout* out) {
  const int G = s->n_q_heads / s->n_kv_heads;
  const long rows = (long)G * (R + nb);
  if (R < 0 || nb < 0 || rows > kMaxRows) return false;
  const int RP = (int)(((rows + 31) / 32) * 32);
  const size_t units = (size_t)s->n_seq * s->n_kv_heads;
  out->RP = RP;
  out->select = kHeaderBytes;
  size_t off = select_end(s);
  out->obs = off;
  off = align256(off + units * RP * s->head_dim * elem_bytes(s->dtype));
  out->valid = off;
  off = align256(off + units * RP * sizeof(int32_t));
  out->lse = off;
  off = align256(off + units * RP * sizeof(float));
  out->rope = off;
  off = align256(off + (size_t)s->n_seq * (R + 1) * (s->head_dim / 2) * sizeof(float2));
  out->beacons = off;
  off = align256(off + (size_t)s->n_seq * s->n_q_heads * (nb + 1) * sizeof(int32_t));
  out->beacon_rows = off;
  off = align256(off + (size_t)s->n_seq * s->n_q_heads * nb * s->head_dim * elem_bytes(s->dtype));
  out->total = off;
  return true;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return BKV_E_WORKSPACE;
  if (((uintptr_t)ws & 255) != 0) return BKV_E_WORKSPACE;
  if (ws_bytes < need) return BKV_E_WORKSPACE;
  return BKV_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BKV_OK : BKV_E_HIP; }

// Argument checks of the scoring calls, in a fixed order (the first failing
// check decides the status).  qbuf and qcount are only checked for non-null,
// and only when the call runs the beacon FPS itself; C < 0 means the call
// takes no capacity (nb is then only range-checked).
int check_score_args(const bkv_shape* shape, const void* K, const int32_t* len, const void* recent,
                     const int32_t* recent_pos, int32_t R, const void* qbuf, const int32_t* qcount, bool need_qcount,
                     int32_t C, int32_t nb, const int32_t* pos_now, double rope_theta, const float* scores,
                     const void* ws, size_t ws_bytes, WsLayout* w) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (C >= 0 ? (C < 2 || C > kMaxCapacity || nb < 0 || nb > C) : (nb < 0 || nb > kMaxCapacity))
    return BKV_E_CAPACITY;
  if (R < 0 || R > kMaxRecent) return BKV_E_SHAPE;
  if (!(rope_theta > 1.0)) return BKV_E_SHAPE;
  if (!layout(shape, R, nb, w)) return BKV_E_SHAPE;
  if (w->RP == 0) return BKV_E_SHAPE;  // no observation rows at all
  if (!K || !len || !scores || !pos_now || (need_qcount && (!qbuf || !qcount))) return BKV_E_NULL;
  if (R > 0 && (!recent || !recent_pos)) return BKV_E_NULL;
  return check_ws(ws, ws_bytes, w->total);
}


}  // namespace

// Whether the scoring calls also write the rotated observation rows to the
// workspace (process-wide; off unless bkv_set_debug_copies turned it on).
static std::atomic<int> g_debug_copies{0};
static bool debug_copies_on() { return g_debug_copies.load(std::memory_order_relaxed) != 0; }

// The RoPE tables and the score kernel, with the beacon picks already in ws.
int enqueue_score(const bkv_shape* shape, const void* K, const int32_t* len, const void* recent,
                  const int32_t* recent_pos, int32_t R, int32_t nb, const int32_t* pos_now, double rope_theta,
                  float* scores, void* ws, const WsLayout& w, bool mean, hipStream_t stream,
                  const float* capture = nullptr) {
  const int N = shape->n_seq, Hq = shape->n_q_heads, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  unsigned char* base = (unsigned char*)ws;
  int32_t* words = (int32_t*)ws;
  float2* tab = (float2*)(base + w.rope);
  void* obs = debug_copies_on() ? base + w.obs : nullptr;  // null: the kernel skips the copy
  int32_t* valid = (int32_t*)(base + w.valid);
  float* lse = (float*)(base + w.lse);
  const int32_t* beacons = (const int32_t*)(base + w.beacons);
  const void* brows = base + w.beacon_rows;
  hipError_t e;
#define BKV_SCORE_CASE(DT, D)                                                                                  \
  e = launch_score<DT, D>(K, len, N, Hkv, Hq, shape->max_len, recent, recent_pos, R, beacons, brows, nb,       \
                          pos_now, rope_theta, tab, obs, valid, w.RP, scores, lse, words, mean, capture, stream);
  if (shape->dtype == BKV_BF16) {
    if (shape->head_dim == 128) {
      BKV_SCORE_CASE(BKV_BF16, 128)
    } else {
      BKV_SCORE_CASE(BKV_BF16, 64)
    }
  } else {
    if (shape->head_dim == 128) {
      BKV_SCORE_CASE(BKV_F32, 128)
    } else {
      BKV_SCORE_CASE(BKV_F32, 64)
    }
  }
#undef BKV_SCORE_CASE
  return hip_status(e);
}
}  // namespace bkv

using namespace bkv;

extern "C" {

size_t bkv_workspace_size(const bkv_shape* shape, int32_t R, int32_t nb) {
  if (check_shape(shape) != BKV_OK) return 0;
  WsLayout w;
  if (!layout(shape, R, nb, &w)) return 0;
  return w.total;
}

int bkv_workspace_layout(const bkv_shape* shape, int32_t R, int32_t nb, size_t offsets[7]) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (!offsets) return BKV_E_NULL;
  WsLayout w;
  if (!layout(shape, R, nb, &w)) return BKV_E_SHAPE;
  offsets[0] = w.obs;
  offsets[1] = w.valid;
  offsets[2] = w.lse;
  offsets[3] = w.select;
  offsets[4] = w.rope;
  offsets[5] = w.beacons;
  offsets[6] = w.beacon_rows;
  return BKV_OK;
}

int bkv_fps_update(const bkv_shape* shape, const void* q_new, int32_t T, void* qbuf, int32_t* qcount, int32_t C,
                   int32_t M, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (C < 2 || C > kMaxCapacity || M < 1 || M >= C) return BKV_E_CAPACITY;
  if (T < 0) return BKV_E_SHAPE;
  if (!qbuf || !qcount || (T > 0 && !q_new)) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, kHeaderBytes)) != BKV_OK) return st;
  const int heads = shape->n_seq * shape->n_q_heads;
  if (heads == 0) return BKV_OK;
  int32_t* w = (int32_t*)ws;
  hipError_t e;
  if (shape->dtype == BKV_BF16)
    e = shape->head_dim == 128 ? launch_fps_update<BKV_BF16, 128>(q_new, T, qbuf, qcount, C, M, heads, w, stream)
                               : launch_fps_update<BKV_BF16, 64>(q_new, T, qbuf, qcount, C, M, heads, w, stream);
  else
    e = shape->head_dim == 128 ? launch_fps_update<BKV_F32, 128>(q_new, T, qbuf, qcount, C, M, heads, w, stream)
                               : launch_fps_update<BKV_F32, 64>(q_new, T, qbuf, qcount, C, M, heads, w, stream);
  return hip_status(e);
}

size_t bkv_fps_full_workspace_size(const bkv_shape* shape, int32_t n) {
  if (check_shape(shape) != BKV_OK || n < 0 || n > kMaxHistory) return 0;
  return fps_full_workspace_bytes((long)shape->n_seq * shape->n_q_heads, n, shape->head_dim);
}

int bkv_fps_full(const bkv_shape* shape, const void* hist, int32_t n, int32_t k, int32_t* picks, void* ws,
                 size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (n < 0 || n > kMaxHistory || k < 0 || k > kMaxFullPicks) return BKV_E_SHAPE;
  const long heads = (long)shape->n_seq * shape->n_q_heads;
  if (heads == 0 || k == 0) return BKV_OK;
  if (!picks || (n > 0 && !hist)) return BKV_E_NULL;
  if (n > 0 && ((uintptr_t)hist & 15u) != 0) return BKV_E_SHAPE;
  if (heads * (((long)n + 1023) / 1024) > INT32_MAX || heads > INT32_MAX) return BKV_E_SHAPE;  // grid size
  if ((st = check_ws(ws, ws_bytes, bkv_fps_full_workspace_size(shape, n))) != BKV_OK) return st;
  hipError_t e;
  if (shape->dtype == BKV_BF16)
    e = shape->head_dim == 128 ? launch_fps_full<BKV_BF16, 128>(hist, heads, n, k, picks, ws, stream)
                               : launch_fps_full<BKV_BF16, 64>(hist, heads, n, k, picks, ws, stream);
  else
    e = shape->head_dim == 128 ? launch_fps_full<BKV_F32, 128>(hist, heads, n, k, picks, ws, stream)
                               : launch_fps_full<BKV_F32, 64>(hist, heads, n, k, picks, ws, stream);
  return hip_status(e);
}

int bkv_beacon_picks(const bkv_shape* shape, const void* qbuf, const int32_t* qcount, int32_t C, int32_t R,
                     int32_t nb, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (C < 2 || C > kMaxCapacity || nb < 0 || nb > C) return BKV_E_CAPACITY;
  if (R < 0 || R > kMaxRecent) return BKV_E_SHAPE;
  WsLayout w;
  if (!layout(shape, R, nb, &w)) return BKV_E_SHAPE;
  if (!qbuf || !qcount) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, w.total)) != BKV_OK) return st;
  const int heads = shape->n_seq * shape->n_q_heads;
  if (heads == 0) return BKV_OK;
  int32_t* words = (int32_t*)ws;
  int32_t* beacons = (int32_t*)((unsigned char*)ws + w.beacons);
  void* brows = (unsigned char*)ws + w.beacon_rows;
  hipError_t e;
#define BKV_PICKS(DT, D) launch_beacon_picks<DT, D>(qbuf, qcount, C, nb, heads, beacons, brows, words, stream)
  if (shape->dtype == BKV_BF16)
    e = shape->head_dim == 128 ? BKV_PICKS(BKV_BF16, 128) : BKV_PICKS(BKV_BF16, 64);
  else
    e = shape->head_dim == 128 ? BKV_PICKS(BKV_F32, 128) : BKV_PICKS(BKV_F32, 64);
#undef BKV_PICKS
  return hip_status(e);
}

int bkv_score_picked(const bkv_shape* shape, const void* K, const int32_t* len, const void* recent,
                     const int32_t* recent_pos, int32_t R, int32_t nb, const int32_t* pos_now, double rope_theta,
                     float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  WsLayout w;
  int st = check_score_args(shape, K, len, recent, recent_pos, R, nullptr, nullptr, false, -1, nb, pos_now,
                            rope_theta, scores, ws, ws_bytes, &w);
  if (st != BKV_OK) return st;
  return enqueue_score(shape, K, len, recent, recent_pos, R, nb, pos_now, rope_theta, scores, ws, w, false, stream);
}

int bkv_score_picked_agg(const bkv_shape* shape, const void* K, const int32_t* len, const void* recent,
                         const int32_t* recent_pos, int32_t R, int32_t nb, const int32_t* pos_now, double rope_theta,
                         int32_t aggregation, float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (aggregation != BKV_AGG_MAX && aggregation != BKV_AGG_MEAN) return BKV_E_SHAPE;
  WsLayout w;
  int st = check_score_args(shape, K, len, recent, recent_pos, R, nullptr, nullptr, false, -1, nb, pos_now,
                            rope_theta, scores, ws, ws_bytes, &w);
  if (st != BKV_OK) return st;
  return enqueue_score(shape, K, len, recent, recent_pos, R, nb, pos_now, rope_theta, scores, ws, w,
                       aggregation == BKV_AGG_MEAN, stream);
}

int bkv_score_picked_capture(const bkv_shape* shape, const void* K, const int32_t* len, const float* capture,
                             int32_t nb, const int32_t* pos_now, double rope_theta, float* scores, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  WsLayout w;
  int st = check_score_args(shape, K, len, nullptr, nullptr, 0, nullptr, nullptr, false, -1, nb, pos_now, rope_theta,
                            scores, ws, ws_bytes, &w);
  if (st != BKV_OK) return st;
  if (!capture) return BKV_E_NULL;
  return enqueue_score(shape, K, len, nullptr, nullptr, 0, nb, pos_now, rope_theta, scores, ws, w, false, stream,
                       capture);
}

size_t bkv_decode_workspace_size(const bkv_shape* shape) {
  if (check_shape(shape) != BKV_OK) return 0;
  const size_t G = (size_t)(shape->n_q_heads / shape->n_kv_heads);
  return align256(kHeaderBytes) + align256((size_t)shape->n_seq * shape->n_kv_heads * G * shape->max_len * 4);
}

int bkv_decode_attention(const bkv_shape* shape, const void* q, const void* K, const void* V, const int32_t* len,
                         float* out, float* capture, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  const int G = shape->n_q_heads / shape->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 5 && G != 8) return BKV_E_SHAPE;
  if (!q || !K || !V || !len || !out) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, capture ? bkv_decode_workspace_size(shape) : kHeaderBytes)) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  int32_t* words = (int32_t*)ws;
  float* logits = capture ? (float*)((unsigned char*)ws + align256(kHeaderBytes)) : nullptr;
  hipError_t e;
#define BKV_DEC(DT, D) launch_decode<DT, D>(q, K, V, len, N, Hkv, G, shape->max_len, out, capture, logits, words, stream)
  if (shape->dtype == BKV_BF16)
    e = shape->head_dim == 128 ? BKV_DEC(BKV_BF16, 128) : BKV_DEC(BKV_BF16, 64);
  else
    e = shape->head_dim == 128 ? BKV_DEC(BKV_F32, 128) : BKV_DEC(BKV_F32, 64);
#undef BKV_DEC
  return hip_status(e);
}

int bkv_beacon_rows(const bkv_shape* shape, const void* src, int32_t S, const int32_t* idx, int32_t R, int32_t nb,
                    void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (nb < 0 || nb > kMaxCapacity) return BKV_E_CAPACITY;
  if (R < 0 || R > kMaxRecent || S < 0) return BKV_E_SHAPE;
  WsLayout w;
  if (!layout(shape, R, nb, &w)) return BKV_E_SHAPE;
  if ((nb > 0 && !idx) || (S > 0 && nb > 0 && !src)) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, w.total)) != BKV_OK) return st;
  const int heads = shape->n_seq * shape->n_q_heads;
  if (heads == 0) return BKV_OK;
  unsigned char* base = (unsigned char*)ws;
  return hip_status(launch_beacon_rows(src, S, idx, nb, shape->head_dim * elem_bytes(shape->dtype), heads,
                                       (int32_t*)(base + w.beacons), base + w.beacon_rows, (int32_t*)ws, stream));
}

int bkv_score(const bkv_shape* shape, const void* K, const int32_t* len, const void* recent,
              const int32_t* recent_pos, int32_t R, const void* qbuf, const int32_t* qcount, int32_t C, int32_t nb,
              const int32_t* pos_now, double rope_theta, float* scores, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  WsLayout w;
  int st = check_score_args(shape, K, len, recent, recent_pos, R, qbuf, qcount, true, C, nb, pos_now, rope_theta,
                            scores, ws, ws_bytes, &w);
  if (st != BKV_OK) return st;  // nothing enqueued
  st = bkv_beacon_picks(shape, qbuf, qcount, C, R, nb, ws, ws_bytes, stream);
  if (st != BKV_OK) return st;
  return enqueue_score(shape, K, len, recent, recent_pos, R, nb, pos_now, rope_theta, scores, ws, w, false, stream);
}

int bkv_select(const bkv_shape* shape, const float* scores, const int32_t* len, int32_t budget, int32_t window,
               int32_t* kept, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (window < 0 || budget < window || budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!scores || !len || !kept) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, select_end(shape))) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  int32_t* words = (int32_t*)ws;
  int32_t* sel = (int32_t*)((unsigned char*)ws + kHeaderBytes);
  return hip_status(launch_select(scores, len, N, Hkv, shape->max_len, budget, window, kept, sel, words, stream));
}

int bkv_compact(const bkv_shape* shape, void* K, void* V, int32_t* len, int32_t budget, const int32_t* kept,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!K || !V || !len || !kept) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, select_end(shape))) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  const int32_t* sel = (const int32_t*)((unsigned char*)ws + kHeaderBytes);
  unsigned long long* moved = (unsigned long long*)((unsigned char*)ws + 8);
  const int row_bytes = shape->head_dim * elem_bytes(shape->dtype);
  return hip_status(launch_compact(K, V, kept, sel, len, N, Hkv, shape->max_len, budget, row_bytes, moved, stream));
}

int bkv_select_compact(const bkv_shape* shape, const float* scores, void* K, void* V, int32_t* len, int32_t budget,
                       int32_t window, int32_t* kept, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = bkv_select(shape, scores, len, budget, window, kept, ws, ws_bytes, stream);
  if (st != BKV_OK) return st;
  return bkv_compact(shape, K, V, len, budget, kept, ws, ws_bytes, stream);
}

int bkv_select_compact_noalloc(const bkv_shape* shape, const float* scores, void* K, void* V, int32_t* len,
                               int32_t budget, int32_t window, int32_t* kept, int32_t* dev_status,
                               hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (window < 0 || budget < window || budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!scores || !K || !V || !len || !kept) return BKV_E_NULL;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if ((long)N * Hkv > kNoallocMaxUnits) return BKV_E_SCRATCH;
  if (N == 0) return BKV_OK;
  unsigned char* base = nullptr;
  if ((st = scratch_on_current_device(&base)) != BKV_OK) return st;
  int32_t* words = (int32_t*)base;
  int32_t* sel = (int32_t*)(base + kHeaderBytes);
  unsigned long long* moved = (unsigned long long*)(base + 8);
  // the previous call's status and statistics are cleared by a kernel (no
  // memset node, so the call can be captured into a graph)
  hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, stream, words);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = launch_select(scores, len, N, Hkv, shape->max_len, budget, window, kept, sel, words, stream);
  if (e == hipSuccess) {
    const int row_bytes = shape->head_dim * elem_bytes(shape->dtype);
    e = launch_compact(K, V, kept, sel, len, N, Hkv, shape->max_len, budget, row_bytes, moved, stream);
  }
  if (e == hipSuccess && dev_status) {
    hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, stream, (const int32_t*)words, dev_status);
    e = hipGetLastError();
  }
  return hip_status(e);
}

int bkv_select_fill(const bkv_shape* shape, const float* scores, const int32_t* pos, const int32_t* len,
                    int32_t budget, int32_t window, int32_t* kept, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (window < 0 || budget < window || budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!scores || !pos || !len || !kept) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, select_end(shape))) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  int32_t* words = (int32_t*)ws;
  int32_t* sel = (int32_t*)((unsigned char*)ws + kHeaderBytes);
  return hip_status(
      launch_select_fill(scores, pos, len, N, Hkv, shape->max_len, budget, window, kept, sel, words, stream));
}

int bkv_compact_fill(const bkv_shape* shape, void* K, void* V, int32_t* pos, int32_t* len, int32_t budget,
                     const int32_t* kept, void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!K || !V || !pos || !len || !kept) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, select_end(shape))) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  int32_t* sel = (int32_t*)((unsigned char*)ws + kHeaderBytes);
  unsigned long long* moved = (unsigned long long*)((unsigned char*)ws + 8);
  const int row_bytes = shape->head_dim * elem_bytes(shape->dtype);
  return hip_status(
      launch_compact_fill(K, V, pos, kept, sel, len, N, Hkv, shape->max_len, budget, row_bytes, moved, stream));
}

int bkv_select_compact_fill(const bkv_shape* shape, const float* scores, void* K, void* V, int32_t* pos,
                            int32_t* len, int32_t budget, int32_t window, int32_t* kept, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  int st = check_shape(shape);
  if (st != BKV_OK) return st;
  if (window < 0 || budget < window || budget < 1 || budget > shape->max_len) return BKV_E_BUDGET;
  if (!scores || !K || !V || !pos || !len || !kept) return BKV_E_NULL;
  if ((st = check_ws(ws, ws_bytes, select_end(shape))) != BKV_OK) return st;
  const int N = shape->n_seq, Hkv = shape->n_kv_heads;
  if (N == 0) return BKV_OK;
  int32_t* words = (int32_t*)ws;
  int32_t* sel = (int32_t*)((unsigned char*)ws + kHeaderBytes);
  unsigned long long* moved = (unsigned long long*)((unsigned char*)ws + 8);
  const int row_bytes = shape->head_dim * elem_bytes(shape->dtype);
  return hip_status(launch_select_compact_fill(scores, K, V, pos, len, N, Hkv, shape->max_len, budget, window, kept,
                                               sel, row_bytes, moved, words, stream));
}

const char* bkv_status_string(int status) {
  switch (status) {
    case BKV_OK: return "ok";
    case BKV_E_NULL: return "a required pointer is NULL";
    case BKV_E_SHAPE: return "a size or count is outside the supported range";
    case BKV_E_DTYPE: return "unsupported storage type";
    case BKV_E_BUDGET: return "budget and window are inconsistent (need 0 <= window <= budget <= max_len)";
    case BKV_E_CAPACITY: return "buffer capacity, shrink target or beacon count out of range";
    case BKV_E_WORKSPACE: return "workspace NULL, too small or not 256-byte aligned";
    case BKV_E_HIP: return "a HIP kernel launch failed";
    case BKV_E_SCRATCH:
      return "n_seq * n_kv_heads exceeds the 131,040 (slot, KV head) units the static scratch of "
             "bkv_select_compact_noalloc holds";
    default: return "unknown status";
  }
}

int bkv_read_device_status(const void* ws, int32_t* status_out, hipStream_t stream) {
  if (!ws || !status_out) return BKV_E_NULL;
  hipError_t e = hipMemcpyAsync(status_out, ws, sizeof(int32_t), hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  return hip_status(e);
}

int32_t bkv_set_debug_copies(int32_t on) { return g_debug_copies.exchange(on != 0 ? 1 : 0) != 0 ? 1 : 0; }

int bkv_reset_device_status(void* ws, hipStream_t stream) {
  if (!ws) return BKV_E_NULL;
  if (((uintptr_t)ws & 255) != 0) return BKV_E_WORKSPACE;
  hipLaunchKernelGGL(zero_header_kernel, dim3(1), dim3(64), 0, stream, (int32_t*)ws);
  return hip_status(hipGetLastError());
}

}  // extern "C"

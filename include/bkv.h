/*
 * bkv.h -- C ABI of libbkv, the BeaconKV eviction hot path for AMD MI355X
 * (gfx950).
 *
 * BeaconKV keeps, per attention head, a small set of "beacon" queries chosen
 * by farthest point sampling from the head's query history, and scores the
 * KV cache with the attention of the recent queries together with those
 * beacons before evicting down to a budget.  Sources (web pages about the
 * method, cited by title and section):
 *   [WZ] wzjinhao.cn news article 56682 on BeaconKV, sections
 *        "怎么挑出这几个信标" (FPS, Continual FPS, pre-RoPE similarity) and
 *        "信标查询怎么用" (beacon positions, max aggregation);
 *   [IK] inkeast.github.io MessageDaily paper-reading post on BeaconKV,
 *        section 三 (I = TopK(score(K,V), B_KV)) and section 4.4;
 *   [AM] aimodeling.com "BeaconKV: Beacon Queries Fix KV Eviction for Long
 *        Reasoning", section "Beacon queries anticipate what will be
 *        revisited" (recent window always kept; 16 beacons, 16 recent
 *        queries, window 32 by default).
 *
 * Conventions for every entry point
 *   - Every pointer except `shape` and `status_out` is a DEVICE pointer on the
 *     current HIP device.  The caller owns and allocates every buffer,
 *     including the workspace; the library never allocates, frees or
 *     synchronises (bkv_read_device_status excepted) and keeps no state
 *     between calls, except for the one scratch array per device of
 *     bkv_select_compact_noalloc, which takes no workspace, and the
 *     process-wide debug-copy switch (bkv_set_debug_copies).
 *   - Work is enqueued on `stream` (0 = the null stream), in call order.
 *   - Tensors are dense and row-major in the index order written next to
 *     them.  N = shape->n_seq, Hkv = shape->n_kv_heads, Hq =
 *     shape->n_q_heads (a multiple of Hkv; G = Hq / Hkv), d =
 *     shape->head_dim, Lmax = shape->max_len.  Storage element type of K, V
 *     and every query tensor: shape->dtype.  Query head g belongs to KV head
 *     g / G.
 *   - The return value is a synchronous status from host-side argument
 *     checks (BKV_E_*), or BKV_E_HIP if a launch failed; nothing is enqueued
 *     when it is not BKV_OK.  Data-dependent violations found on the device
 *     (a length above Lmax, a buffer count outside [0, C)) set bits of the
 *     device status word in the workspace and the affected unit is left
 *     untouched; read it with bkv_read_device_status.
 *   - Calls that share a workspace must not run concurrently, with two
 *     exceptions.  bkv_fps_update only ORs bits into the status word, so it
 *     may overlap any call that does not use its buffers (bkv_score_picked
 *     and the selection and compaction calls do not).  bkv_beacon_picks
 *     writes only workspace regions [5] and [6] and the status word, so it
 *     may overlap bkv_select* and bkv_compact*; it must still come after the
 *     bkv_score_picked that reads the previous picks (an event, as for any
 *     cross-stream dependency).
 */
#ifndef BKV_H
#define BKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bkv_status {
  BKV_OK = 0,
  BKV_E_NULL = 1,      /* a required pointer is NULL */
  BKV_E_SHAPE = 2,     /* a size or count is outside the supported range */
  BKV_E_DTYPE = 3,     /* unsupported storage type */
  BKV_E_BUDGET = 4,    /* budget < window, window < 0 or budget > max_len */
  BKV_E_CAPACITY = 5,  /* shrink target not in [1, C), or capacity too large */
  BKV_E_WORKSPACE = 6, /* workspace NULL, too small or not 256-byte aligned */
  BKV_E_HIP = 7,       /* a kernel launch failed */
  BKV_E_SCRATCH = 8    /* bkv_select_compact_noalloc: more units than its scratch holds */
};

enum bkv_dtype { BKV_F32 = 0, BKV_BF16 = 1 };

/* Device status bits (bkv_read_device_status). */
#define BKV_DEV_BAD_LEN 0x1   /* len[n] < 0 or len[n] > max_len */
#define BKV_DEV_BAD_COUNT 0x2 /* qcount[n][g] < 0 or >= C on entry */
#define BKV_DEV_BAD_INDEX 0x4 /* bkv_beacon_rows: a row index >= S */

/* Aggregation of the observation rows' probabilities into a key's score. */
enum bkv_aggregation { BKV_AGG_MAX = 0, BKV_AGG_MEAN = 1 };

/* Supported ranges (checked on the host):
 *   head_dim in {64, 128}; C (buffer capacity) <= 256; G * (R + nb) <= 256;
 *   R <= 64; nb <= C; max_len <= 1 << 24. */

typedef struct bkv_shape {
  int32_t n_seq;      /* N: sequence slots (e.g. layers x batch, flattened) */
  int32_t n_kv_heads; /* Hkv */
  int32_t n_q_heads;  /* Hq, a multiple of Hkv */
  int32_t head_dim;   /* d */
  int32_t max_len;    /* Lmax: rows allocated per (slot, KV head) in K and V */
  int32_t dtype;      /* enum bkv_dtype */
} bkv_shape;

/*
 * Workspace.  One byte buffer, 256-byte aligned, at least
 * bkv_workspace_size(shape, R, nb) bytes, serves every call made with the
 * same shape, R and nb.  It holds the device status word (int32 at offset 0),
 * run statistics (uint64 rows_moved at offset 8: rows gathered by
 * bkv_compact since the last reset), and the per-call intermediates whose
 * offsets bkv_workspace_layout reports:
 *   [0] obs     : rotated observation rows [N][Hkv][RP][d], storage type,
 *                 RP = G*(R+nb) rounded up to 32; row g*(R+nb)+r holds recent
 *                 query r of query head h*G+g, row g*(R+nb)+R+b its beacon b;
 *                 absent rows are zero.  Written by the scoring calls only
 *                 while debug copies are on (bkv_set_debug_copies), else left
 *                 as it was;
 *   [1] valid   : int32 [N][Hkv][RP], 1 for present rows;
 *   [2] lse     : float [N][Hkv][RP], natural-log row normaliser of the
 *                 softmax (+inf for absent rows);
 *   [3] select  : int32 [N][Hkv][2] = {first evicted index, kept count};
 *   [4] rope    : float2 [N][R+1][d/2] (cos, sin) tables;
 *   [5] beacons : int32 [N][Hq][nb+1]: the pick count, then the buffer rows
 *                 of the beacons in pick order;
 *   [6] beacon rows : [N][Hq][nb][d], storage type: copies of the picked
 *                 buffer rows (pre-RoPE), the first `count` of each head valid.
 * Zero the first 256 bytes once before first use (bkv_reset_device_status).
 */
size_t bkv_workspace_size(const bkv_shape *shape, int32_t R, int32_t nb);
int bkv_workspace_layout(const bkv_shape *shape, int32_t R, int32_t nb, size_t offsets[7]);

/*
 * bkv_fps_update -- Continual FPS ingest ([WZ] 怎么挑出这几个信标: a bounded
 * buffer per attention head, compressed by FPS back to a smaller size
 * whenever it fills; [AM]: sampling in pre-RoPE query space).
 *
 *   q_new  [N][Hq][T][d]  new pre-RoPE queries, oldest first (read only)
 *   qbuf   [N][Hq][C][d]  per-query-head buffers (in/out); rows [0, count)
 *                         are live: retained FPS picks first, then arrivals
 *                         in time order
 *   qcount [N][Hq]        live row count, in [0, C) on entry (in/out)
 *   C, M                  capacity and shrink target, 1 <= M < C <= 256
 *   T >= 0                queries per head in this call
 *
 * The T queries are appended one at a time; each time the count reaches C
 * the buffer is replaced by its FPS picks (M of them, in pick order).  FPS on
 * cosine similarity: start at the row with the lowest mean cosine to all
 * rows, then repeatedly add the row whose maximum cosine to the picked set
 * is lowest; ties go to the lower row.  Cosines are evaluated in binary64.
 * Rows at or beyond the final count are unspecified.  Query rows must be
 * finite; with non-finite rows the picks are unspecified, though always rows
 * of the buffer (the same holds for the beacon FPS of the scoring calls).
 */
int bkv_fps_update(const bkv_shape *shape, const void *q_new, int32_t T, void *qbuf,
                   int32_t *qcount, int32_t C, int32_t M, void *ws, size_t ws_bytes,
                   hipStream_t stream);

/*
 * bkv_score -- beacon-guided importance scores ([IK] 三 and 4.4; [WZ]
 * 信标查询怎么用).
 *
 *   K          [N][Hkv][Lmax][d]  cached keys, stored after RoPE (read only)
 *   len        [N]                cache length L of each slot, <= Lmax
 *   recent     [N][Hq][R][d]      recent pre-RoPE queries, R >= 0
 *   recent_pos [N][R]             their positions; a negative position marks
 *                                 an absent query
 *   qbuf, qcount, C               the buffers of bkv_fps_update (read only)
 *   nb                            beacons per query head (0 <= nb <= C)
 *   pos_now    [N]                position of the current decode step
 *   rope_theta                    RoPE base
 *   scores     [N][Hkv][Lmax]     output, float; entries j < L are written
 *
 * For every query head the beacons are FPS(qbuf[0..count), min(nb, count)).
 * Beacons are rotated to pos_now, recent queries to their own positions
 * (rotate-half RoPE, inverse frequency theta^(-2i/d) held in binary32, angle
 * in binary64, cos/sin held in binary32, rotation in binary64, result rounded
 * once to the storage type).  Every observation row r of the G query heads
 * of a KV head attends to all L keys: p_r = softmax_j(q_r . k_j / sqrt(d)),
 * and score_j = max_r p_r(j).  Without any present row the scores are 0.
 */
int bkv_score(const bkv_shape *shape, const void *K, const int32_t *len, const void *recent,
              const int32_t *recent_pos, int32_t R, const void *qbuf, const int32_t *qcount,
              int32_t C, int32_t nb, const int32_t *pos_now, double rope_theta, float *scores,
              void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * bkv_score in two calls, so that the beacon FPS can run on another stream.
 * After bkv_beacon_picks the buffers are free: the next ingest may run while
 * bkv_score_picked still scores (for instance on a second stream, during the
 * current eviction).
 *
 * bkv_beacon_picks -- the beacon FPS of every query head (the first half of
 *   bkv_score): writes workspace regions [5] (pick count, then the buffer
 *   rows of the picks) and [6] (copies of the picked rows).  qbuf, qcount,
 *   C, nb as for bkv_score; R only locates the regions (the workspace of
 *   shape, R, nb).
 *
 * bkv_score_picked -- the second half: rotation and scoring exactly as
 *   bkv_score, with the beacons taken from regions [5] and [6] as the last
 *   bkv_beacon_picks on this workspace left them.  Reads no buffer.
 *
 * bkv_score = bkv_beacon_picks followed by bkv_score_picked on one stream.
 */
int bkv_beacon_picks(const bkv_shape *shape, const void *qbuf, const int32_t *qcount, int32_t C,
                     int32_t R, int32_t nb, void *ws, size_t ws_bytes, hipStream_t stream);
int bkv_score_picked(const bkv_shape *shape, const void *K, const int32_t *len, const void *recent,
                     const int32_t *recent_pos, int32_t R, int32_t nb, const int32_t *pos_now,
                     double rope_theta, float *scores, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/*
 * Policy variants on the same kernels, for the comparisons the pages make
 * ([WZ] 效果到底怎么样: InitialRecent keeps the earliest generated queries
 * with the recent ones, and loses to the FPS beacons; [IK] 4.4: a key's score
 * aggregates the rows' attention by maximum or mean, and [WZ] 信标查询怎么用
 * uses the maximum).
 *
 * bkv_beacon_rows -- beacons given instead of chosen by FPS: writes regions
 *   [5] and [6] as bkv_beacon_picks does, for bkv_score_picked(_agg) to use.
 *     src  [N][Hq][S][d]  rows to take beacons from (read only): e.g. qbuf
 *                         (S = C) for representatives drawn at random, or
 *                         a caller-kept copy of each head's first queries
 *                         for InitialRecent
 *     idx  [N][Hq][nb]    int32 rows of src, in beacon order; the beacons of
 *                         a head are its leading entries in [0, S): the first
 *                         negative entry ends them, as does an entry >= S,
 *                         which also sets BKV_DEV_BAD_INDEX
 *   R and nb locate the regions (the workspace of shape, R, nb); 0 <= nb <=
 *   256, S >= 0.  No beacons at all (recent queries only) is nb = 0, or idx
 *   all -1.
 *
 * bkv_score_picked_agg -- bkv_score_picked with a choice of aggregation:
 *   BKV_AGG_MAX (bkv_score_picked itself) or BKV_AGG_MEAN, the mean of the
 *   rows' probabilities over the rows present in the (slot, KV head) (0 if
 *   none).  Everything else as bkv_score_picked.
 */
int bkv_beacon_rows(const bkv_shape *shape, const void *src, int32_t S, const int32_t *idx, int32_t R,
                    int32_t nb, void *ws, size_t ws_bytes, hipStream_t stream);
int bkv_score_picked_agg(const bkv_shape *shape, const void *K, const int32_t *len, const void *recent,
                         const int32_t *recent_pos, int32_t R, int32_t nb, const int32_t *pos_now,
                         double rope_theta, int32_t aggregation, float *scores, void *ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * bkv_select -- kept set ([IK] 三: I = TopK(score, B_KV); [AM]: the recent
 * window is always kept).
 *
 *   scores [N][Hkv][Lmax]  non-negative finite floats, j < len[n] read
 *   len    [N]             current lengths (read only)
 *   budget, window         B_KV (window included) and W, 0 <= W <= B_KV <= Lmax
 *   kept   [N][Hkv][B_KV]  output: ascending kept indices
 *
 * If L <= B_KV every index is kept (kept[i] = i for i < L, -1 after).
 * Otherwise kept = [L-W, L) plus the B_KV-W highest scores of [0, L-W),
 * ties at the cut going to the lower index.  Selection is exact on the
 * binary32 scores.  Also records, per (slot, KV head), the first evicted
 * index and the kept count in the workspace for bkv_compact.
 */
int bkv_select(const bkv_shape *shape, const float *scores, const int32_t *len, int32_t budget,
               int32_t window, int32_t *kept, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * bkv_compact -- in-place, order-preserving gather of the kept rows.
 *
 *   K, V [N][Hkv][Lmax][d]  in/out; row i <- row kept[i] for i < kept count
 *                           (bit copies of the pre-call rows); rows at or
 *                           beyond the kept count are left as they were
 *   len  [N]                set to min(len, budget)
 *   kept                    the output of bkv_select with the same workspace
 *
 * Must follow bkv_select on the same workspace, budget and stream.  Adds the
 * number of moved rows (per tensor) to the workspace statistic rows_moved.
 * One workgroup per (slot, KV head, tensor) moves its rows in increasing
 * index order, in steps of 128 KB; no workgroup waits for another.
 */
int bkv_compact(const bkv_shape *shape, void *K, void *V, int32_t *len, int32_t budget,
                const int32_t *kept, void *ws, size_t ws_bytes, hipStream_t stream);

/* bkv_select followed by bkv_compact. */
int bkv_select_compact(const bkv_shape *shape, const float *scores, void *K, void *V,
                       int32_t *len, int32_t budget, int32_t window, int32_t *kept, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * bkv_select_compact_noalloc -- bkv_select_compact for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): no workspace argument; the same
 * selection and compaction kernels use a scratch array the library holds in
 * device memory, 1 MiB per device for the life of the process (status word,
 * statistics, and the select table of at most 131,040 (slot, KV head)
 * units).
 *
 *   scores, K, V, len, budget, window, kept  as bkv_select_compact
 *   dev_status  int32 DEVICE pointer or NULL: receives this call's device
 *               status word (BKV_DEV_* bits; 0 when every unit was valid)
 *
 * Results equal bkv_select_compact's.  Returns BKV_E_SCRATCH (nothing
 * enqueued) when n_seq * n_kv_heads > 131,040.  Every call on a device uses
 * that device's one scratch array: calls that overlap on one device (on
 * different streams, or from several host threads without ordering) race and
 * must not be issued.  Each call clears the status word first; the select
 * table is fully rewritten by the selection before the compaction reads it.
 * Allocates and frees nothing; the first call on a device looks up the
 * array's device address (hipGetSymbolAddress).
 */
int bkv_select_compact_noalloc(const bkv_shape *shape, const float *scores, void *K, void *V,
                               int32_t *len, int32_t budget, int32_t window, int32_t *kept,
                               int32_t *dev_status, hipStream_t stream);

/*
 * Hole-filling layout.  The order-preserving compaction above moves every
 * kept row after the first evicted one.  In this layout the rows need not be
 * in position order: each row carries its token position, and eviction only
 * moves the kept rows that lie at or beyond the budget into the evicted rows
 * below it.  The kept set is the one bkv_select computes when the rows are
 * in position order (same sources: [IK] 三, TopK of the scores; [AM], the
 * recent window always kept), with the window and the tie order stated by
 * position instead of by row.
 *
 * bkv_select_fill
 *   scores [N][Hkv][Lmax]  non-negative finite floats, j < len[n] read
 *   pos    [N][Hkv][Lmax]  int32 token position of each row, j < len[n] read;
 *                          positions are expected to be distinct per (slot,
 *                          KV head) (equal ones are ordered by row)
 *   len    [N]             current lengths (read only)
 *   budget, window         B_KV (window included) and W, 0 <= W <= B_KV <= Lmax
 *   kept   [N][Hkv][B_KV]  output gather map: after compaction row i holds
 *                          the pre-eviction row kept[i]
 *
 * If L <= B_KV every row is kept (kept[i] = i for i < L, -1 after).
 * Otherwise the window is the W rows of highest position (ties: lower row)
 * and the other B_KV - W kept rows are the highest scores among the rest
 * (ties: lower position, then lower row).  The evicted rows of [0, B_KV),
 * ascending, are paired with the kept rows of [B_KV, L), ascending:
 * kept[i] = i for a kept row i < B_KV, else its partner.  Selection is exact
 * on the binary32 scores.  Records the first evicted row below B_KV and the
 * kept count in the workspace for bkv_compact_fill.
 */
int bkv_select_fill(const bkv_shape *shape, const float *scores, const int32_t *pos,
                    const int32_t *len, int32_t budget, int32_t window, int32_t *kept, void *ws,
                    size_t ws_bytes, hipStream_t stream);

/*
 * bkv_compact_fill -- in-place hole filling.
 *
 *   K, V [N][Hkv][Lmax][d]  in/out; row i <- row kept[i] for every i below
 *                           the kept count with kept[i] != i (bit copies);
 *                           all other rows are left as they were
 *   pos  [N][Hkv][Lmax]     in/out; moved with the rows
 *   len  [N]                set to min(len, budget)
 *   kept                    the output of bkv_select_fill with the same
 *                           workspace
 *
 * Must follow bkv_select_fill on the same workspace, budget and stream.
 * Adds the number of moved K and V rows to the statistic rows_moved, and
 * leaves the select table reading "no hole", so a repeated call moves
 * nothing.
 */
int bkv_compact_fill(const bkv_shape *shape, void *K, void *V, int32_t *pos, int32_t *len,
                     int32_t budget, const int32_t *kept, void *ws, size_t ws_bytes,
                     hipStream_t stream);

/* bkv_select_fill followed by bkv_compact_fill, with the same results (also
 * the select table reading "no hole").  Where max_len <= 4096 one kernel
 * selects and fills: each (slot, KV head) moves its fillers as soon as it
 * has paired them. */
int bkv_select_compact_fill(const bkv_shape *shape, const float *scores, void *K, void *V,
                            int32_t *pos, int32_t *len, int32_t budget, int32_t window,
                            int32_t *kept, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Recent-query scores captured during decoding ([WZ] 信标查询怎么用: the score
 * of a key takes the attention of the recent queries with the beacons';
 * [WZ] 信标和最近查询该怎么分配: the beacons' attention is the extra cost).
 * Decoding computes every recent query's attention anyway, so its
 * probabilities can be kept as they are produced, and at eviction only the
 * beacons need a scoring pass.  A captured probability is normalised over the
 * keys present at its own decode step (the eviction-time rows of bkv_score
 * are normalised over the whole cache).
 *
 * bkv_decode_attention -- one decode step of attention for every query head:
 *     q       [N][Hq][d]     the step's queries, already rotated (read only)
 *     K, V    [N][Hkv][Lmax][d]  the cache, rows [0, len[n]) present
 *     len     [N]            int32, in [0, Lmax] (else BKV_DEV_BAD_LEN, unit
 *                            untouched)
 *     out     [N][Hq][d]     float: softmax_j(q . k_j / sqrt(d)) v_j summed
 *                            over the present keys; 0 when len = 0
 *     capture [N][Hkv][Lmax] float or NULL: for j < len[n],
 *                            capture[j] = max(capture[j], max_g p_g(j)) over
 *                            the G query heads of the KV head; the caller
 *                            zeroes it where the recent window starts
 *   ws: its own workspace, 256-byte aligned: bkv_decode_workspace_size(shape)
 *   bytes with a capture array (the step's logits are staged there), 256
 *   without.  G = Hq / Hkv in {1, 2, 4, 5, 8}.
 *
 * bkv_score_picked_capture -- the eviction scores from the beacons alone
 *   (bkv_score_picked with R = 0: the workspace of shape, 0, nb, after
 *   bkv_beacon_picks with R = 0), each key's score then raised to its
 *   captured recent maximum: scores[j] = max(beacon score, capture[j]).
 */
size_t bkv_decode_workspace_size(const bkv_shape *shape);
int bkv_decode_attention(const bkv_shape *shape, const void *q, const void *K, const void *V,
                         const int32_t *len, float *out, float *capture, void *ws, size_t ws_bytes,
                         hipStream_t stream);
int bkv_score_picked_capture(const bkv_shape *shape, const void *K, const int32_t *len,
                             const float *capture, int32_t nb, const int32_t *pos_now, double rope_theta,
                             float *scores, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * bkv_fps_full -- FPS over each query head's WHOLE stored history: the naive
 * alternative that Continual FPS replaces ([WZ] 怎么挑出这几个信标: FPS over
 * every past query would keep the full history of each head, which the
 * bounded buffer avoids).  For comparing the two; not a step of the
 * eviction pass.
 *
 *   hist   [N][Hq][n][d]  the first n pre-RoPE queries of every query head,
 *                         16-byte aligned (read only)
 *   n      >= 0, <= 1 << 24
 *   k      0 <= k <= 4096 picks per head
 *   picks  [N][Hq][k]     int32 out: row indices in pick order; entries from
 *                         min(k, n) on are -1
 *   ws     its own workspace, 256-byte aligned, at least
 *          bkv_fps_full_workspace_size(shape, n) bytes (row norms, running
 *          maximum cosines, per-chunk partial results); no status word
 *
 * The picking rule is bkv_fps_update's (lowest mean cosine start, then the
 * row with the lowest maximum cosine to the picked set, ties to the lower
 * row, norms clamped at 1e-12), evaluated in binary64; the mean cosine of a
 * row is its dot product with the sum of the normalised rows, divided by its
 * norm and n.  Every pick reads the whole history once: min(k, n) + 1
 * passes over hist.  Rows must be finite (with non-finite rows the picks
 * are unspecified, though still inside [0, n)).  Only shape->n_seq,
 * n_q_heads, head_dim and dtype are used.
 */
size_t bkv_fps_full_workspace_size(const bkv_shape *shape, int32_t n);
int bkv_fps_full(const bkv_shape *shape, const void *hist, int32_t n, int32_t k, int32_t *picks,
                 void *ws, size_t ws_bytes, hipStream_t stream);

/* Text for a bkv_status value (static string). */
const char *bkv_status_string(int status);

/* Copies the device status word to *status_out; synchronises `stream`. */
int bkv_read_device_status(const void *ws, int32_t *status_out, hipStream_t stream);

/* Zeroes the status word and statistics (first 256 bytes of ws) on `stream`. */
int bkv_reset_device_status(void *ws, hipStream_t stream);

/*
 * Debug copies: while on (on != 0), the scoring calls (bkv_score,
 * bkv_score_picked, bkv_score_picked_agg, bkv_score_picked_capture) also
 * write the rotated observation rows they score with to the workspace
 * region [0] obs, for checking the rotation; off by default, since the
 * scores do not need them (at 4,608 units of 128 rows, d = 128 bf16, they
 * are 151 MB of writes per call).  Process-wide, for calls enqueued after it
 * returns; returns the previous setting (0 or 1).  Enqueues nothing.
 */
int32_t bkv_set_debug_copies(int32_t on);

#ifdef __cplusplus
}
#endif

#endif /* BKV_H */

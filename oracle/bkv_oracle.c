/*
 * bkv_oracle.c -- plain, slow, single-threaded CPU oracle of the BeaconKV
 * eviction hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product path (the
 * HIP library and its Python binding) never calls it, and the two share no
 * code, header, table or constant.
 *
 * Every computation is carried out in IEEE binary64 unless a step below says
 * otherwise.  Storage types are binary32 ("f32") and bfloat16 ("bf16", held as
 * its 16-bit pattern).
 *
 * Sources (the method is described on web pages, cited by title and section):
 *   [WZ]  wzjinhao.cn news article 56682 on BeaconKV (Chinese), sections
 *         "怎么挑出这几个信标" (how the beacons are picked: FPS, Continual FPS,
 *         pre-RoPE space) and "信标查询怎么用" (how beacon queries are used:
 *         positions, max aggregation).
 *   [IK]  inkeast.github.io MessageDaily paper-reading post on BeaconKV,
 *         section 三 (problem definition: I = TopK(score(K,V), B_KV)) and
 *         section 4.4 (beacon-guided eviction).
 *   [AM]  aimodeling.com "BeaconKV: Beacon Queries Fix KV Eviction for Long
 *         Reasoning", section "Beacon queries anticipate what will be
 *         revisited" (recent sliding window always kept; defaults 16/16/32).
 *
 * Readings taken where the pages are silent are listed next to each step.
 *
 * Parity status: every function below is pinned by the CPU test suite
 * (brute force, closed forms, invariants and library routines); none is
 * "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

/* ------------------------------------------------------------------------ */
/* Storage conversions                                                        */
/* ------------------------------------------------------------------------ */

/* Exact widening of one stored element to binary64. */
double orc_load(const void *base, int dtype, long idx) {
  if (dtype == ORC_F32) {
    return (double)((const float *)base)[idx];
  }
  uint16_t h = ((const uint16_t *)base)[idx];
  uint32_t w = (uint32_t)h << 16; /* bf16 is the top half of a binary32 */
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* Round a binary64 value once, to nearest with ties to even, to bfloat16
 * (8 significant bits, binary32 exponent range, gradual underflow).  Written
 * from the format's definition: scale by the bf16 spacing at |v|, round to an
 * integer in the default (nearest-even) mode, scale back. */
uint16_t orc_bf16_from_double(double v) {
  if (isnan(v)) return (uint16_t)0x7FC0;
  if (isinf(v)) return v > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
  if (v == 0.0) return signbit(v) ? (uint16_t)0x8000 : (uint16_t)0x0000;
  int e;
  (void)frexp(v, &e);            /* |v| = f * 2^e, f in [0.5, 1) */
  int q = e - 8;                 /* spacing of 8-bit significands at |v| */
  if (q < -133) q = -133;        /* bf16 subnormal spacing is 2^-133 */
  double r = nearbyint(ldexp(v, -q)); /* exact scaling, then RNE */
  double out = ldexp(r, q);
  if (fabs(out) >= 0x1p128) return v > 0 ? (uint16_t)0x7F80 : (uint16_t)0xFF80;
  float f = (float)out;          /* exactly representable, no rounding */
  uint32_t w;
  memcpy(&w, &f, sizeof w);
  return (uint16_t)(w >> 16);
}

/* Store v into a storage element with a single rounding from binary64. */
void orc_store(void *base, int dtype, long idx, double v) {
  if (dtype == ORC_F32) {
    ((float *)base)[idx] = (float)v; /* C conversion rounds to nearest-even */
  } else {
    ((uint16_t *)base)[idx] = orc_bf16_from_double(v);
  }
}

static size_t elem_size(int dtype) { return dtype == ORC_F32 ? 4 : 2; }

/* ------------------------------------------------------------------------ */
/* Farthest point sampling on cosine similarity                               */
/* ------------------------------------------------------------------------ */

static double dot(const double *a, const double *b, int d) {
  double s = 0.0;
  for (int t = 0; t < d; ++t) s += a[t] * b[t];
  return s;
}

/*
 * orc_fps: greedy farthest point sampling of up to k of the c vectors X[c][d].
 * [WZ, 怎么挑出这几个信标]: start at the query whose mean similarity to all
 * queries is lowest; then, round after round, add the remaining query that is
 * least similar to (farthest from) the already-selected set, until the preset
 * number is reached.  Similarity is cosine similarity.
 *
 * Readings: the distance of a point to the selected set is its distance to
 * the nearest selected point, so "least similar to the set" means the lowest
 * maximum cosine to the set.  The mean similarity includes the point itself.
 * Ties go to the lowest index.  Norms are clamped at 1e-12 (a zero vector has
 * cosine 0 with everything).  If c <= k every vector is returned.
 *
 * Returns the number of picks, min(k, c), written to picks[] in pick order.
 */
int orc_fps(const double *X, int c, int d, int k, int *picks) {
  int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  double *xh = (double *)malloc(sizeof(double) * (size_t)c * d);
  double *m = (double *)malloc(sizeof(double) * c);
  char *picked = (char *)calloc(c, 1);

  /* normalise every vector */
  for (int i = 0; i < c; ++i) {
    double n = sqrt(dot(X + (size_t)i * d, X + (size_t)i * d, d));
    if (n < 1e-12) n = 1e-12;
    for (int t = 0; t < d; ++t) xh[(size_t)i * d + t] = X[(size_t)i * d + t] / n;
  }

  /* start: lowest mean cosine similarity to all c vectors */
  int start = -1;
  double best_mu = 0.0;
  for (int i = 0; i < c; ++i) {
    double sum = 0.0;
    for (int j = 0; j < c; ++j) sum += dot(xh + (size_t)i * d, xh + (size_t)j * d, d);
    double mu = sum / c;
    if (start < 0 || mu < best_mu) {
      start = i;
      best_mu = mu;
    }
  }
  if (start < 0) start = 0; /* unreachable for c >= 1; keeps the index provably valid */
  picks[0] = start;
  picked[start] = 1;
  for (int i = 0; i < c; ++i) m[i] = dot(xh + (size_t)i * d, xh + (size_t)start * d, d);

  /* greedy rounds: the unpicked vector with the lowest max-cosine to the set */
  for (int t = 1; t < kk; ++t) {
    int best = -1;
    for (int i = 0; i < c; ++i) {
      if (picked[i]) continue;
      if (best < 0 || m[i] < m[best]) best = i;
    }
    if (best < 0) best = 0; /* unreachable: kk <= c leaves an unpicked row */
    picks[t] = best;
    picked[best] = 1;
    for (int i = 0; i < c; ++i) {
      double s = dot(xh + (size_t)i * d, xh + (size_t)best * d, d);
      if (s > m[i]) m[i] = s;
    }
  }
  free(xh);
  free(m);
  free(picked);
  return kk;
}

/*
 * orc_fps_objectives: the quantity FPS minimises in a round, for every row of
 * X[c][d], given the rows already picked (prefix[0..np)).  With an empty
 * prefix it is the mean cosine to all c rows (the start rule); otherwise the
 * maximum cosine to the picked rows (the farthest-point rule).  Same
 * definitions and readings as orc_fps.  It lets a test check that a pick
 * sequence is a valid FPS run when exact ties make several sequences valid.
 */
void orc_fps_objectives(const double *X, int c, int d, const int *prefix, int np, double *out) {
  double *xh = (double *)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1) * d);
  for (int i = 0; i < c; ++i) {
    double n = sqrt(dot(X + (size_t)i * d, X + (size_t)i * d, d));
    if (n < 1e-12) n = 1e-12;
    for (int t = 0; t < d; ++t) xh[(size_t)i * d + t] = X[(size_t)i * d + t] / n;
  }
  for (int i = 0; i < c; ++i) {
    if (np == 0) {
      double sum = 0.0;
      for (int j = 0; j < c; ++j) sum += dot(xh + (size_t)i * d, xh + (size_t)j * d, d);
      out[i] = sum / c;
    } else {
      double m = -INFINITY;
      for (int k = 0; k < np; ++k) {
        double s = dot(xh + (size_t)i * d, xh + (size_t)prefix[k] * d, d);
        if (s > m) m = s;
      }
      out[i] = m;
    }
  }
  free(xh);
}

/*
 * orc_fps_stored: FPS over the first c rows of a stored buffer (row stride d).
 * The rows are widened exactly to binary64 first.
 */
int orc_fps_stored(const void *buf, int dtype, int c, int d, int k, int *picks) {
  if (c <= 0) return 0;
  double *X = (double *)malloc(sizeof(double) * (size_t)c * d);
  for (long i = 0; i < (long)c * d; ++i) X[i] = orc_load(buf, dtype, i);
  int n = orc_fps(X, c, d, k, picks);
  free(X);
  return n;
}

/*
 * orc_fps_full: FPS over a head's whole stored query history buf[c][d], the
 * naive alternative that Continual FPS replaces.
 * [WZ, 怎么挑出这几个信标]: running FPS over every query seen so far would mean
 * keeping the full history of each head; the bounded, repeatedly compressed
 * buffer exists to avoid exactly that.  The picking rule and its readings are
 * orc_fps's: start at the lowest mean cosine similarity (self included), then
 * take the unpicked row with the lowest maximum cosine to the picked ones,
 * ties to the lowest index, norms clamped at 1e-12.
 *
 * The start rule's mean similarity of row i is evaluated as
 * x^_i . (sum_j x^_j) / c.  By linearity of the dot product this is the
 * pairwise mean of orc_fps (rounding order aside), in O(c*d) instead of
 * O(c^2*d) operations, which keeps histories of tens of thousands of queries
 * tractable.  Rows are widened exactly to binary64 first.
 *
 * Returns min(k, c) picks, written to picks[] in pick order.
 */
static double *normalised_rows(const void *buf, int dtype, int c, int d) {
  double *xh = (double *)malloc(sizeof(double) * (size_t)(c > 0 ? c : 1) * d);
  for (int i = 0; i < c; ++i) {
    double *r = xh + (size_t)i * d;
    for (int t = 0; t < d; ++t) r[t] = orc_load(buf, dtype, (long)i * d + t);
    double n = sqrt(dot(r, r, d));
    if (n < 1e-12) n = 1e-12;
    for (int t = 0; t < d; ++t) r[t] /= n;
  }
  return xh;
}

/* Mean cosine similarity of every row to all c rows, via the summed row. */
static void mean_similarity(const double *xh, int c, int d, double *mu) {
  double *sum = (double *)calloc((size_t)d, sizeof(double));
  for (int j = 0; j < c; ++j)
    for (int t = 0; t < d; ++t) sum[t] += xh[(size_t)j * d + t];
  for (int i = 0; i < c; ++i) mu[i] = dot(xh + (size_t)i * d, sum, d) / c;
  free(sum);
}

int orc_fps_full(const void *buf, int dtype, int c, int d, int k, int *picks) {
  int kk = k < c ? k : c;
  if (kk <= 0) return 0;
  double *xh = normalised_rows(buf, dtype, c, d);
  double *m = (double *)malloc(sizeof(double) * c);
  char *picked = (char *)calloc(c, 1);

  mean_similarity(xh, c, d, m);
  int start = 0;
  for (int i = 1; i < c; ++i)
    if (m[i] < m[start]) start = i;
  picks[0] = start;
  picked[start] = 1;
  for (int i = 0; i < c; ++i) m[i] = dot(xh + (size_t)i * d, xh + (size_t)start * d, d);

  for (int t = 1; t < kk; ++t) {
    int best = -1;
    for (int i = 0; i < c; ++i) {
      if (picked[i]) continue;
      if (best < 0 || m[i] < m[best]) best = i;
    }
    if (best < 0) best = 0; /* unreachable: kk <= c leaves an unpicked row */
    picks[t] = best;
    picked[best] = 1;
    for (int i = 0; i < c; ++i) {
      double s = dot(xh + (size_t)i * d, xh + (size_t)best * d, d);
      if (s > m[i]) m[i] = s;
    }
  }
  free(xh);
  free(m);
  free(picked);
  return kk;
}

/*
 * orc_fps_full_objectives: orc_fps_objectives for a stored history, with the
 * start rule's mean similarity evaluated as in orc_fps_full.  out[i] is the
 * mean cosine of row i to all c rows for an empty prefix, else its maximum
 * cosine to the picked rows prefix[0..np).
 */
void orc_fps_full_objectives(const void *buf, int dtype, int c, int d, const int *prefix, int np, double *out) {
  double *xh = normalised_rows(buf, dtype, c, d);
  if (np == 0) {
    mean_similarity(xh, c, d, out);
  } else {
    for (int i = 0; i < c; ++i) {
      double m = -INFINITY;
      for (int q = 0; q < np; ++q) {
        double s = dot(xh + (size_t)i * d, xh + (size_t)prefix[q] * d, d);
        if (s > m) m = s;
      }
      out[i] = m;
    }
  }
  free(xh);
}

/*
 * orc_fps_ingest: Continual FPS for one attention head.
 * [WZ, 怎么挑出这几个信标]: each attention head keeps only a small buffer with
 * an upper bound on its size; once the buffer is full an FPS pass compresses
 * it back to a smaller size, and the cycle repeats, so the full query history
 * is never stored.  [AM, "Beacon queries anticipate what will be revisited"]:
 * sampling works on pre-RoPE queries.
 *
 * Readings: every decode query of the head enters the buffer in time order;
 * "full" means the count reaches C right after an append; the shrunk buffer
 * holds the M picked rows (original stored values, bit copies) in pick order,
 * and later arrivals follow them.
 *
 * buf: [C][d] storage rows; *count in [0, C) on entry; q_new: [T][d] rows.
 * Returns 0, or -1 if the entry count or the sizes are invalid (buf untouched).
 */
int orc_fps_ingest(void *buf, int dtype, int d, int C, int M, int *count,
                   const void *q_new, int T) {
  int c = *count;
  if (c < 0 || c >= C || M < 1 || M >= C || d < 1 || T < 0) return -1;
  size_t es = elem_size(dtype);
  size_t row = es * (size_t)d;
  char *b = (char *)buf;
  const char *q = (const char *)q_new;
  int *picks = (int *)malloc(sizeof(int) * M);
  char *tmp = (char *)malloc(row * (size_t)M);
  for (int t = 0; t < T; ++t) {
    memcpy(b + row * c, q + row * t, row);
    c += 1;
    if (c == C) {
      int n = orc_fps_stored(buf, dtype, C, d, M, picks);
      for (int i = 0; i < n; ++i) memcpy(tmp + row * i, b + row * picks[i], row);
      memcpy(b, tmp, row * (size_t)n);
      c = n;
    }
  }
  free(picks);
  free(tmp);
  *count = c;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding                                                  */
/* ------------------------------------------------------------------------ */

/*
 * orc_rope: rotate one pre-RoPE vector x[d] to position pos.
 * The pages name RoPE without fixing a convention.  Reading (the convention
 * of Qwen3-family models): rotate-half pairing of coordinates i and i + d/2,
 * inverse frequency theta^(-2i/d) evaluated in binary64 and held as binary32,
 * angle pos * freq in binary64 (exact), cos and sin evaluated in binary64 and
 * held as binary32, rotation evaluated in binary64.  The caller rounds y once
 * to the storage type.
 */
void orc_rope(const double *x, int d, long pos, double theta, double *y) {
  int h = d / 2;
  for (int i = 0; i < h; ++i) {
    double freq = (double)(float)pow(theta, -(2.0 * i) / (double)d);
    double a = (double)pos * freq;
    double cs = (double)(float)cos(a);
    double sn = (double)(float)sin(a);
    y[i] = x[i] * cs - x[i + h] * sn;
    y[i + h] = x[i + h] * cs + x[i] * sn;
  }
}

/* ------------------------------------------------------------------------ */
/* Beacon-guided scoring of one (sequence slot, KV head)                      */
/* ------------------------------------------------------------------------ */

/* One observation row: a stored pre-RoPE query rotated to position pos and
 * rounded once to the storage type (reading R8), widened back to binary64. */
static void rotated_row(const char *src, int dtype, int d, long pos, double theta, double *x, double *yr,
                        double *out) {
  for (int t = 0; t < d; ++t) x[t] = orc_load(src, dtype, t);
  orc_rope(x, d, pos, theta, yr);
  for (int t = 0; t < d; ++t) {
    char cell[4];
    orc_store(cell, dtype, 0, yr[t]);
    out[t] = orc_load(cell, dtype, 0);
  }
}

#define ORC_AGG_MAX 0
#define ORC_AGG_MEAN 1

/*
 * score_rows: logits of the present observation rows y[rows][d] against the L
 * stored keys (q.k / sqrt(d), binary64), each row's log-sum-exp over all L
 * keys, and the aggregate over rows of every key's softmax probability:
 * the maximum (ORC_AGG_MAX) or the mean over the present rows
 * (ORC_AGG_MEAN).  No present row gives scores 0; absent rows get lse +inf.
 */
static void score_rows(int dtype, int d, int rows, const double *y, const int *valid, const void *K, int L,
                       int agg, double *scores, double *lse_r) {
  double *s = (double *)malloc(sizeof(double) * (size_t)(rows > 0 ? rows : 1) * (L > 0 ? L : 1));
  double *kj = (double *)malloc(sizeof(double) * d);
  double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int j = 0; j < L; ++j) {
    for (int t = 0; t < d; ++t) kj[t] = orc_load(K, dtype, (long)j * d + t);
    for (int r = 0; r < rows; ++r) {
      if (!valid[r]) continue;
      s[(size_t)r * L + j] = dot(y + (size_t)r * d, kj, d) * inv_sqrt_d;
    }
  }
  int present = 0;
  for (int r = 0; r < rows; ++r) {
    if (!valid[r] || L == 0) {
      lse_r[r] = INFINITY;
      continue;
    }
    present += 1;
    double mx = -INFINITY;
    for (int j = 0; j < L; ++j)
      if (s[(size_t)r * L + j] > mx) mx = s[(size_t)r * L + j];
    double sum = 0.0;
    for (int j = 0; j < L; ++j) sum += exp(s[(size_t)r * L + j] - mx);
    lse_r[r] = mx + log(sum);
  }
  for (int j = 0; j < L; ++j) {
    double best = 0.0, total = 0.0;
    for (int r = 0; r < rows; ++r) {
      if (!valid[r]) continue;
      double p = exp(s[(size_t)r * L + j] - lse_r[r]);
      if (p > best) best = p;
      total += p;
    }
    scores[j] = agg == ORC_AGG_MEAN ? (present > 0 ? total / present : 0.0) : best;
  }
  free(s);
  free(kj);
}

/*
 * orc_score_unit: importance scores of the L cached keys of one KV head.
 *
 * [IK, 三]: eviction keeps I = TopK(score(K,V), B_KV) and BeaconKV's score is
 * the aggregated attention of the recent queries together with the beacon
 * set.  [WZ, 信标查询怎么用]: beacons receive the position encoding of the
 * current decode step, recent queries keep the positions where they were
 * generated, and scores are aggregated by maximum, not mean.
 * [WZ, 怎么挑出这几个信标] and the page glossary: beacons are the queries FPS
 * selects from the head's query history.
 *
 * Readings: one query buffer per query head; the beacons of a query head are
 * FPS(buffer[0..count), nb) at scoring time (min(nb, count) of them); each
 * observation row attends to all L keys (no causal mask), logits are
 * q.k / sqrt(d) on the stored (post-RoPE) keys, softmax is per row over the L
 * keys, and the score of key j is the maximum over all rows of every query
 * head in the KV head's GQA group of that row's softmax probability.  A
 * recent row with a negative position is absent.  If no row is present the
 * scores are 0.  Rotated rows are rounded once to the storage type.
 *
 * Layouts: K [L][d]; recent [G][R][d]; recent_pos [R]; qbuf [G][C][d];
 * qcount [G].  Outputs: scores [L] (binary64); optional obs [G*(R+nb)][d]
 * storage rows (row g*(R+nb)+r for recent r, g*(R+nb)+R+b for beacon b;
 * absent rows zero), obs_valid [G*(R+nb)], lse [G*(R+nb)] (absent rows get
 * +inf).  Returns 0, or -1 for an invalid qcount.
 */
int orc_score_unit(int dtype, int d, int G, const void *K, int L,
                   const void *recent, const int *recent_pos, int R,
                   const void *qbuf, const int *qcount, int C, int nb,
                   long pos_now, double theta, double *scores, void *obs,
                   int *obs_valid, double *lse) {
  int rows = G * (R + nb);
  size_t es = elem_size(dtype);
  double *y = (double *)calloc((size_t)(rows > 0 ? rows : 1) * d, sizeof(double));
  int *valid = (int *)calloc(rows > 0 ? rows : 1, sizeof(int));
  double *x = (double *)malloc(sizeof(double) * d);
  double *yr = (double *)malloc(sizeof(double) * d);
  int *picks = (int *)malloc(sizeof(int) * (nb > 0 ? nb : 1));
  double *lse_r = (double *)malloc(sizeof(double) * (rows > 0 ? rows : 1));
  int status = 0;

  for (int g = 0; g < G; ++g) {
    /* recent queries at their own positions */
    for (int r = 0; r < R; ++r) {
      int row = g * (R + nb) + r;
      if (recent_pos[r] < 0) continue;
      const char *src = (const char *)recent + es * (size_t)d * ((size_t)g * R + r);
      rotated_row(src, dtype, d, recent_pos[r], theta, x, yr, y + (size_t)row * d);
      valid[row] = 1;
    }
    /* beacons: FPS over the buffer, rotated to the current decode position */
    int cnt = qcount[g];
    if (cnt < 0 || cnt >= C) {
      status = -1;
      continue;
    }
    const char *hb = (const char *)qbuf + es * (size_t)d * (size_t)C * g;
    int nsel = orc_fps_stored(hb, dtype, cnt, d, nb, picks);
    for (int b = 0; b < nsel; ++b) {
      int row = g * (R + nb) + R + b;
      const char *src = hb + es * (size_t)d * picks[b];
      rotated_row(src, dtype, d, pos_now, theta, x, yr, y + (size_t)row * d);
      valid[row] = 1;
    }
  }

  score_rows(dtype, d, rows, y, valid, K, L, ORC_AGG_MAX, scores, lse_r);

  if (obs) {
    for (int r = 0; r < rows; ++r)
      for (int t = 0; t < d; ++t) orc_store(obs, dtype, (long)r * d + t, y[(size_t)r * d + t]);
  }
  if (obs_valid)
    for (int r = 0; r < rows; ++r) obs_valid[r] = valid[r];
  if (lse)
    for (int r = 0; r < rows; ++r) lse[r] = lse_r[r];

  free(y);
  free(valid);
  free(x);
  free(yr);
  free(picks);
  free(lse_r);
  return status;
}

/*
 * orc_score_given: orc_score_unit with the beacon rows given instead of
 * chosen by FPS, and a choice of aggregation.  The policy variants the pages
 * compare BeaconKV against run through it:
 *   - [WZ, 效果到底怎么样]: InitialRecent keeps the earliest generated queries
 *     together with the recent ones (the given rows are the first queries);
 *   - representatives drawn at random from the buffer (the given rows are
 *     those draws; the random numbers are the caller's);
 *   - no beacons at all (bcount 0 everywhere, recent queries only);
 *   - [IK, 4.4]: the per-key aggregate over the observation rows may be the
 *     maximum or the mean; [WZ, 信标查询怎么用] takes the maximum.
 * Same readings as orc_score_unit; the mean is over the present rows.
 *
 * Layouts: brows [G][nb][d] storage rows, bcount [G] with 0 <= bcount <= nb
 * (rows [0, bcount[g]) of head g are its beacons).  agg: ORC_AGG_MAX or
 * ORC_AGG_MEAN.  Outputs as orc_score_unit.  Returns 0, or -1 for a bcount
 * outside [0, nb] (that head then has no beacons).
 */
int orc_score_given(int dtype, int d, int G, const void *K, int L, const void *recent, const int *recent_pos, int R,
                    const void *brows, const int *bcount, int nb, long pos_now, double theta, int agg,
                    double *scores, void *obs, int *obs_valid, double *lse) {
  int rows = G * (R + nb);
  size_t es = elem_size(dtype);
  double *y = (double *)calloc((size_t)(rows > 0 ? rows : 1) * d, sizeof(double));
  int *valid = (int *)calloc(rows > 0 ? rows : 1, sizeof(int));
  double *x = (double *)malloc(sizeof(double) * d);
  double *yr = (double *)malloc(sizeof(double) * d);
  double *lse_r = (double *)malloc(sizeof(double) * (rows > 0 ? rows : 1));
  int status = 0;
  for (int g = 0; g < G; ++g) {
    for (int r = 0; r < R; ++r) {
      int row = g * (R + nb) + r;
      if (recent_pos[r] < 0) continue;
      rotated_row((const char *)recent + es * (size_t)d * ((size_t)g * R + r), dtype, d, recent_pos[r], theta, x,
                  yr, y + (size_t)row * d);
      valid[row] = 1;
    }
    int cnt = bcount[g];
    if (cnt < 0 || cnt > nb) {
      status = -1;
      continue;
    }
    for (int b = 0; b < cnt; ++b) {
      int row = g * (R + nb) + R + b;
      rotated_row((const char *)brows + es * (size_t)d * ((size_t)g * nb + b), dtype, d, pos_now, theta, x, yr,
                  y + (size_t)row * d);
      valid[row] = 1;
    }
  }
  score_rows(dtype, d, rows, y, valid, K, L, agg, scores, lse_r);
  if (obs)
    for (int r = 0; r < rows; ++r)
      for (int t = 0; t < d; ++t) orc_store(obs, dtype, (long)r * d + t, y[(size_t)r * d + t]);
  if (obs_valid)
    for (int r = 0; r < rows; ++r) obs_valid[r] = valid[r];
  if (lse)
    for (int r = 0; r < rows; ++r) lse[r] = lse_r[r];
  free(y);
  free(valid);
  free(x);
  free(yr);
  free(lse_r);
  return status;
}

/* ------------------------------------------------------------------------ */
/* Decode attention with the recent rows' probabilities captured              */
/* ------------------------------------------------------------------------ */

/*
 * orc_decode_attention: one decode step of the G query heads of one KV head.
 * Each query q_g (already rotated at its own position) attends to the L
 * cached keys present at this step: p_g(j) = softmax_j(q_g . k_j / sqrt(d)),
 * out_g = sum_j p_g(j) v_j, in binary64.
 *
 * [WZ, 信标查询怎么用] scores keys with the attention of the recent queries;
 * [WZ, 信标和最近查询该怎么分配] places the extra cost of scoring in the
 * beacons' attention.  Reading (R24): a recent query's probabilities can be
 * taken from its own decode step, over the keys present then, instead of
 * being recomputed at eviction time over the whole cache; the per-key
 * aggregate is the maximum over the recent steps and the G heads, as for
 * the eviction-time rows.
 *
 * Layouts: K, V [L][d] storage; q [G][d] storage.  probs [G][L] (binary64,
 * optional), out [G][d] (binary64).  L = 0 gives out = 0.
 */
/* step_probs: p_g(j) = softmax_j(q_g . k_j / sqrt(d)) over the L keys, for
 * the G rows of q, in binary64 (probs [G][L]). */
static void step_probs(int dtype, int d, int G, const void *K, int L, const void *q, double *probs) {
  double *qg = (double *)malloc(sizeof(double) * d);
  double *kj = (double *)malloc(sizeof(double) * d);
  double *s = (double *)malloc(sizeof(double) * (L > 0 ? L : 1));
  double inv_sqrt_d = 1.0 / sqrt((double)d);
  for (int g = 0; g < G; ++g) {
    for (int t = 0; t < d; ++t) qg[t] = orc_load(q, dtype, (long)g * d + t);
    double mx = -INFINITY;
    for (int j = 0; j < L; ++j) {
      for (int t = 0; t < d; ++t) kj[t] = orc_load(K, dtype, (long)j * d + t);
      s[j] = dot(qg, kj, d) * inv_sqrt_d;
      if (s[j] > mx) mx = s[j];
    }
    double sum = 0.0;
    for (int j = 0; j < L; ++j) sum += exp(s[j] - mx);
    for (int j = 0; j < L; ++j) probs[(size_t)g * L + j] = exp(s[j] - mx) / sum;
  }
  free(qg);
  free(kj);
  free(s);
}

void orc_decode_attention(int dtype, int d, int G, const void *K, const void *V, int L, const void *q,
                          double *probs, double *out) {
  double *p = (double *)malloc(sizeof(double) * (size_t)G * (L > 0 ? L : 1));
  step_probs(dtype, d, G, K, L, q, p);
  for (int g = 0; g < G; ++g) {
    for (int t = 0; t < d; ++t) out[(size_t)g * d + t] = 0.0;
    for (int j = 0; j < L; ++j) {
      double pj = p[(size_t)g * L + j];
      if (probs) probs[(size_t)g * L + j] = pj;
      for (int t = 0; t < d; ++t) out[(size_t)g * d + t] += pj * orc_load(V, dtype, (long)j * d + t);
    }
  }
  free(p);
}

/*
 * orc_capture_step: folds one decode step of the G query heads of a KV head
 * into the recent-query capture (reading R24).  [WZ, 信标查询怎么用]: a key's
 * score takes the largest attention any recent query (or beacon) gives it;
 * a recent query's attention is the one of its own decode step, over the L
 * keys present at that step.  capture[j] = max(capture[j], max_g p_g(j)) for
 * j < L; entries at or beyond L are left as they were (the step gives them
 * probability 0).  The caller zeroes the capture where the recent window
 * starts.  q [G][d] storage rows, already rotated at the step's position.
 */
void orc_capture_step(int dtype, int d, int G, const void *K, int L, const void *q, double *capture) {
  double *p = (double *)malloc(sizeof(double) * (size_t)G * (L > 0 ? L : 1));
  step_probs(dtype, d, G, K, L, q, p);
  for (int j = 0; j < L; ++j)
    for (int g = 0; g < G; ++g)
      if (p[(size_t)g * L + j] > capture[j]) capture[j] = p[(size_t)g * L + j];
  free(p);
}

/*
 * orc_score_capture: the eviction score of one KV head when the recent
 * queries' attention was captured during decoding (reading R24): the
 * beacon rows alone are scored at eviction time ([WZ, 信标和最近查询该怎么分配]
 * puts the extra cost of scoring in the beacons' attention), exactly as
 * orc_score_unit with no recent rows, and each key's score is then the larger
 * of that beacon score and its captured value: the maximum over the beacon
 * rows and the captured recent steps, as [WZ, 信标查询怎么用] aggregates.
 * Layouts as orc_score_unit; capture [L] (binary64).  Returns 0, or -1 for an
 * invalid qcount.
 */
int orc_score_capture(int dtype, int d, int G, const void *K, int L, const void *qbuf, const int *qcount, int C,
                      int nb, long pos_now, double theta, const double *capture, double *scores) {
  int status = orc_score_unit(dtype, d, G, K, L, NULL, NULL, 0, qbuf, qcount, C, nb, pos_now, theta, scores, NULL,
                              NULL, NULL);
  for (int j = 0; j < L; ++j)
    if (capture[j] > scores[j]) scores[j] = capture[j];
  return status;
}

/* ------------------------------------------------------------------------ */
/* Selection and compaction                                                   */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  int index;
} scored_t;

static int by_score_desc_index_asc(const void *pa, const void *pb) {
  const scored_t *a = (const scored_t *)pa, *b = (const scored_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->index > b->index) - (a->index < b->index);
}

/*
 * orc_select: the kept set of one KV head.
 * [IK, 三]: at eviction time keep I = TopK(score, B_KV).  [AM, "Beacon queries
 * anticipate what will be revisited"]: keep the top scores; the last W
 * entries (the recent window) are kept whatever their scores.
 *
 * Readings: B_KV counts every kept entry, the window included; the window is
 * the last W entries [L-W, L); the other B-W are the top scores of [0, L-W),
 * ties broken towards the lower index; if L <= B nothing is evicted.
 *
 * kept[] receives min(L, B) indices in ascending order.  Returns that count,
 * or -1 if W > B, W < 0 or B < 0.
 */
int orc_select(const double *scores, int L, int B, int W, int *kept) {
  if (B < 0 || W < 0 || W > B || L < 0) return -1;
  if (L <= B) {
    for (int i = 0; i < L; ++i) kept[i] = i;
    return L;
  }
  int n = L - W;
  scored_t *v = (scored_t *)malloc(sizeof(scored_t) * (n > 0 ? n : 1));
  for (int j = 0; j < n; ++j) {
    v[j].score = scores[j];
    v[j].index = j;
  }
  qsort(v, n, sizeof(scored_t), by_score_desc_index_asc);
  char *keep = (char *)calloc(L, 1);
  for (int i = 0; i < B - W; ++i) keep[v[i].index] = 1;
  for (int j = L - W; j < L; ++j) keep[j] = 1;
  int c = 0;
  for (int j = 0; j < L; ++j)
    if (keep[j]) kept[c++] = j;
  free(v);
  free(keep);
  return c;
}

/*
 * orc_compact: X'[i] = X[kept[i]] for i < n, as bit copies of the rows of the
 * pre-eviction X; rows >= n are left as they were.  The pages only say the
 * kept entries are retained; reading: an order-preserving gather into the
 * front of the same buffer.
 */
void orc_compact(void *X, long row_bytes, const int *kept, int n) {
  char *x = (char *)X;
  char *old = (char *)malloc((size_t)row_bytes * (n > 0 ? n : 1));
  for (int i = 0; i < n; ++i) memcpy(old + (size_t)row_bytes * i, x + (size_t)row_bytes * kept[i], row_bytes);
  memcpy(x, old, (size_t)row_bytes * n);
  free(old);
}

/* ------------------------------------------------------------------------ */
/* Hole-filling layout (positions carried with the rows)                      */
/* ------------------------------------------------------------------------ */

typedef struct {
  double score;
  long pos;
  int row;
} placed_t;

/* Newest first: position descending, then the lower row. */
static int by_pos_desc_row_asc(const void *pa, const void *pb) {
  const placed_t *a = (const placed_t *)pa, *b = (const placed_t *)pb;
  if (a->pos > b->pos) return -1;
  if (a->pos < b->pos) return 1;
  return (a->row > b->row) - (a->row < b->row);
}

/* Highest score first, then the older position, then the lower row. */
static int by_score_desc_pos_asc_row_asc(const void *pa, const void *pb) {
  const placed_t *a = (const placed_t *)pa, *b = (const placed_t *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  if (a->pos < b->pos) return -1;
  if (a->pos > b->pos) return 1;
  return (a->row > b->row) - (a->row < b->row);
}

/*
 * orc_select_fill: the kept set of one KV head when rows are not kept in
 * position order, and the gather map that fills the evicted rows.
 * [IK, 三]: keep I = TopK(score, B_KV); [AM, "Beacon queries anticipate what
 * will be revisited"]: the newest W entries are kept whatever their scores.
 *
 * Readings: row j holds the token at position pos[j].  The window is the W
 * newest tokens, i.e. the first W rows by (position descending, row
 * ascending); the other B-W kept rows are the first ones of the remaining
 * rows by (score descending, position ascending, row ascending).  With
 * positions ascending in the row index this is exactly orc_select's kept set
 * (window = last W rows, ties to the lower index).  Layout after eviction:
 * the rows of [0, B) that are evicted ("holes", ascending) take, in order,
 * the kept rows of [B, L) (ascending), so only those rows move.
 *
 * kept[i] (i < min(L, B)) receives the pre-eviction row that row i holds
 * afterwards: i itself for a kept row below B, else the filling row.
 * Returns min(L, B), or -1 if W > B, W < 0 or B < 0.
 */
int orc_select_fill(const double *scores, const long *pos, int L, int B, int W, int *kept) {
  if (B < 0 || W < 0 || W > B || L < 0) return -1;
  if (L <= B) {
    for (int i = 0; i < L; ++i) kept[i] = i;
    return L;
  }
  placed_t *v = (placed_t *)malloc(sizeof(placed_t) * L);
  for (int j = 0; j < L; ++j) {
    v[j].score = scores[j];
    v[j].pos = pos[j];
    v[j].row = j;
  }
  char *keep = (char *)calloc(L, 1);
  /* the window: the W newest rows */
  qsort(v, L, sizeof(placed_t), by_pos_desc_row_asc);
  for (int i = 0; i < W; ++i) keep[v[i].row] = 1;
  /* the others: top B-W of the rest */
  int n = 0;
  for (int i = W; i < L; ++i) v[n++] = v[i];
  qsort(v, n, sizeof(placed_t), by_score_desc_pos_asc_row_asc);
  for (int i = 0; i < B - W; ++i) keep[v[i].row] = 1;
  /* pair the holes of [0, B) with the kept rows of [B, L), both ascending */
  int next_src = B;
  for (int i = 0; i < B; ++i) {
    if (keep[i]) {
      kept[i] = i;
    } else {
      while (!keep[next_src]) ++next_src;
      kept[i] = next_src++;
    }
  }
  free(v);
  free(keep);
  return B;
}

/*
 * blasst_oracle.c -- plain fp64 CPU oracle for the BLASST skip-softmax attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY. This is the slow, obviously-correct reference the GPU library is
 * checked against. Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
 * load it. It shares no code, header, table or constant with the GPU library, and the GPU
 * library never calls it.
 *
 * Everything is double precision on contiguous row-major arrays; there is no blocking, fusion or
 * reordering beyond what the sources state. Sources, cited by page title and section:
 *
 *   [SS]  "Skip-Softmax" (vLLM-Omni feature design page), section "Algorithm": the running
 *         values m, l, O of the streaming pass, the per-tile test that skips a tile when
 *         exp(tile_max[i] - running_max[i]) < lambda holds for every query row of the tile, its
 *         log-space form tile_max - running_max < ln(lambda), and that a skipped tile's share of
 *         l and O is simply left out.
 *   [BL]  "BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding" (MLSys 2026 talk
 *         notes), section on the proposed algorithm, Eq. 2: the same test written with the
 *         block-local row max and the running row max of tile j.
 *   [HG]  "The Hitchhiker's Guide -- Phase 08", Section 1 (FlashAttention): the definition
 *         softmax(QK^T / sqrt(d)) V, the online-softmax recurrence for m, l, O, the final O / l,
 *         the tiling into B_r query rows by B_c keys visited in ascending key order, and the
 *         log-sum-exp output L = m + log(l).
 *
 * Readings taken where the pages are silent (each is listed in the design notes):
 *   - lambda is clamped to at most 1; lambda = 0 means tau = -infinity and nothing is skipped.
 *   - the comparison is strict (<), as printed.
 *   - the running max the test compares against is the one that already includes the tile
 *     (its left side then lies in (0, 1] as the Skip-Softmax page states). For lambda <= 1 a
 *     skipped tile can never raise the running max, so leaving m, l, O untouched on a skip is the
 *     same as "updating m first"; the code checks that and reports a violation.
 *   - a row that sees no key of the tile (causal mask, or a padded row) votes "skip": its
 *     contribution to that tile is exactly zero.
 *   - a tile that no row of the block can see is not visited and not counted.
 *   - a split of the key range restarts the running state; splits are merged by log-sum-exp.
 */
#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

/* Tile status codes written to tile_status[]. */
#define ORACLE_TILE_KEPT 0
#define ORACLE_TILE_SKIPPED 1
#define ORACLE_TILE_NOT_VISITED 2

/* Error codes. */
#define ORACLE_OK 0
#define ORACLE_BAD_ARG (-1)
#define ORACLE_NO_MEMORY (-2)
#define ORACLE_SKIP_RAISED_MAX (-3)

static double dot(const double *a, const double *b, int n) {
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += a[i] * b[i];
  return s;
}

/*
 * Dense softmax attention for a block of query rows: the definition in [HG] "Why Standard
 * Attention is IO-Bound", written out with the usual max subtraction.
 *   s_rk  = scale * <q_r, k_k>           for keys row_first[r] <= k < row_keys[r]
 *   O_r   = sum_k exp(s_rk - M_r) v_k / sum_k exp(s_rk - M_r),   M_r = max_k s_rk
 *   LSE_r = M_r + ln sum_k exp(s_rk - M_r)
 * A row with no visible key gets O_r = 0 and LSE_r = -inf. row_first may be NULL (every row's
 * first visible key is 0); a sliding window of W keys ending at the row's position gives
 * row_first = position - W + 1.
 *
 * q: n_rows x d_qk, k: n_keys x d_qk, v: n_keys x d_v, o: n_rows x d_v, lse: n_rows.
 */
int oracle_dense_rows(int n_rows, int n_keys, int d_qk, int d_v, const double *q,
                      const double *k, const double *v, const int *row_first,
                      const int *row_keys, double scale, double *o, double *lse) {
  if (n_rows < 0 || n_keys < 0 || d_qk <= 0 || d_v <= 0) return ORACLE_BAD_ARG;
  double *s = (double *)malloc(sizeof(double) * (n_keys > 0 ? n_keys : 1));
  if (!s) return ORACLE_NO_MEMORY;
  for (int r = 0; r < n_rows; ++r) {
    int nk = row_keys[r] < n_keys ? row_keys[r] : n_keys;
    int j0 = row_first && row_first[r] > 0 ? row_first[r] : 0;
    double *orow = o + (size_t)r * d_v;
    for (int c = 0; c < d_v; ++c) orow[c] = 0.0;
    if (nk <= j0) {
      lse[r] = -INFINITY;
      continue;
    }
    double mx = -INFINITY;
    for (int j = j0; j < nk; ++j) {
      s[j] = scale * dot(q + (size_t)r * d_qk, k + (size_t)j * d_qk, d_qk);
      if (s[j] > mx) mx = s[j];
    }
    double z = 0.0;
    for (int j = j0; j < nk; ++j) {
      double p = exp(s[j] - mx);
      z += p;
      const double *vj = v + (size_t)j * d_v;
      for (int c = 0; c < d_v; ++c) orow[c] += p * vj[c];
    }
    for (int c = 0; c < d_v; ++c) orow[c] /= z;
    lse[r] = mx + log(z);
  }
  free(s);
  return ORACLE_OK;
}

/*
 * The tiled BLASST loop for one block of query rows (one "tile row" of B_r rows) over the key
 * range [k_begin, k_end), in tiles of block_c keys starting at k_begin, visited in ascending
 * order ([HG] "FlashAttention Tiling Strategy"). Keys are indexed absolutely: k and v hold at
 * least k_end rows. Row r sees keys with row_first[r] <= index < row_keys[r] (row_first NULL:
 * from index 0).
 *
 * Per tile ([SS] "Algorithm"; [BL] Eq. 2):
 *   1. scores s_rk = scale * <q_r, k_k>; keys the row cannot see score -inf;
 *   2. tile row max mt_r = max_k s_rk; running max including the tile m'_r = max(m_r, mt_r);
 *   3. row margin d_r = mt_r - m'_r (<= 0); tile margin = max over rows that see a key;
 *   4. skip the tile iff every row votes skip: d_r < ln(lambda), or the row sees no key;
 *   5. otherwise the online-softmax update of [HG]:
 *        alpha = exp(m_r - m'_r), p_rk = exp(s_rk - m'_r),
 *        l_r = alpha l_r + sum_k p_rk,  acc_r = alpha acc_r + sum_k p_rk v_k,  m_r = m'_r.
 * At the end O_r = acc_r / l_r and LSE_r = m_r + ln l_r ([HG], Triton sketch's log-sum-exp).
 *
 * Outputs: o (n_rows x d_v), lse, row_max, row_sum (the final m and l); visited and skipped
 * tile counts (added to *visited / *skipped); per tile, if the arrays are non-NULL and the tile
 * index is below max_tiles: tile_status (kept / skipped / not visited) and tile_margin.
 *
 * forced (may be NULL, else max_tiles entries): take each visited tile's decision from
 * forced[tile] (ORACLE_TILE_SKIPPED = skip, anything else = keep) instead of the test. The rest of
 * the pass is unchanged, so this evaluates the method for a given set of decisions; it exists to
 * check a kernel's output when a tile's margin lies so close to ln(lambda) that float rounding
 * decided it the other way. A forced skip may drop a tile holding a new row maximum; the running
 * max then stays where it was, as in the kernel.
 */
int oracle_blasst_rows(int n_rows, int d_qk, int d_v, const double *q, const double *k,
                       const double *v, const int *row_first, const int *row_keys,
                       int k_begin, int k_end,
                       int block_c, double scale, double lambda, double *o, double *lse,
                       double *row_max, double *row_sum, long long *visited, long long *skipped,
                       unsigned char *tile_status, double *tile_margin, int max_tiles,
                       const unsigned char *forced) {
  if (n_rows < 0 || d_qk <= 0 || d_v <= 0 || block_c <= 0 || k_begin < 0 || k_end < k_begin)
    return ORACLE_BAD_ARG;
  if (!(lambda >= 0.0) || isinf(lambda)) return ORACLE_BAD_ARG; /* NaN, negative or infinite */

  /* Threshold in log space ([SS] "Algorithm": the kernel evaluates m~ - m < ln(lambda)). */
  double lam = lambda > 1.0 ? 1.0 : lambda;
  double tau = lam > 0.0 ? log(lam) : -INFINITY;

  size_t rows = (size_t)(n_rows > 0 ? n_rows : 1);
  double *m = (double *)malloc(sizeof(double) * rows);
  double *l = (double *)malloc(sizeof(double) * rows);
  double *mt = (double *)malloc(sizeof(double) * rows);
  double *acc = (double *)calloc(rows * (size_t)d_v, sizeof(double));
  double *s = (double *)malloc(sizeof(double) * rows * (size_t)block_c);
  if (!m || !l || !mt || !acc || !s) {
    free(m); free(l); free(mt); free(acc); free(s);
    return ORACLE_NO_MEMORY;
  }
  for (int r = 0; r < n_rows; ++r) {
    m[r] = -INFINITY;
    l[r] = 0.0;
  }

  int status = ORACLE_OK;
  int tile = 0;
  for (int t0 = k_begin; t0 < k_end; t0 += block_c, ++tile) {
    int t1 = t0 + block_c < k_end ? t0 + block_c : k_end;

    /* A tile that no row can see is not visited. */
    int seen = 0;
    for (int r = 0; r < n_rows; ++r)
      if (row_keys[r] > t0 && (!row_first || row_first[r] < t1)) seen = 1;
    if (!seen) {
      if (tile_status && tile < max_tiles) tile_status[tile] = ORACLE_TILE_NOT_VISITED;
      if (tile_margin && tile < max_tiles) tile_margin[tile] = -INFINITY;
      continue;
    }
    *visited += 1;

    /* Scores, tile row max, and the tile's margin. */
    double margin = -INFINITY;
    for (int r = 0; r < n_rows; ++r) {
      double *sr = s + (size_t)r * block_c;
      int vis_end = row_keys[r] < t1 ? row_keys[r] : t1;
      int vis_begin = row_first ? row_first[r] : 0;
      mt[r] = -INFINITY;
      for (int kk = t0; kk < t1; ++kk) {
        if (kk >= vis_begin && kk < vis_end) {
          sr[kk - t0] = scale * dot(q + (size_t)r * d_qk, k + (size_t)kk * d_qk, d_qk);
          if (sr[kk - t0] > mt[r]) mt[r] = sr[kk - t0];
        } else {
          sr[kk - t0] = -INFINITY;
        }
      }
      if (mt[r] > -INFINITY) {
        double m_new = m[r] > mt[r] ? m[r] : mt[r];
        double d_r = mt[r] - m_new;
        if (d_r > margin) margin = d_r;
      }
    }
    if (tile_margin && tile < max_tiles) tile_margin[tile] = margin;

    /* The skip test: every row's margin below ln(lambda) (rows without a key vote skip).
       margin is the largest row margin, so "all rows below tau" is "margin < tau". */
    int skip = margin < tau;
    if (forced && tile < max_tiles) skip = forced[tile] == ORACLE_TILE_SKIPPED;
    if (skip) {
      *skipped += 1;
      if (tile_status && tile < max_tiles) tile_status[tile] = ORACLE_TILE_SKIPPED;
      /* With lambda <= 1 a skipped tile cannot hold a new row maximum. */
      if (!forced)
        for (int r = 0; r < n_rows; ++r)
          if (mt[r] > m[r]) status = ORACLE_SKIP_RAISED_MAX;
      continue;
    }
    if (tile_status && tile < max_tiles) tile_status[tile] = ORACLE_TILE_KEPT;

    /* Online-softmax update of [HG] for the kept tile. */
    for (int r = 0; r < n_rows; ++r) {
      double m_new = m[r] > mt[r] ? m[r] : mt[r];
      if (m_new == -INFINITY) continue; /* the row has seen no key yet: nothing to add */
      double alpha = exp(m[r] - m_new);  /* exp(-inf) = 0 on the row's first keys */
      double *ar = acc + (size_t)r * d_v;
      const double *sr = s + (size_t)r * block_c;
      l[r] *= alpha;
      for (int c = 0; c < d_v; ++c) ar[c] *= alpha;
      for (int kk = t0; kk < t1; ++kk) {
        if (sr[kk - t0] == -INFINITY) continue;
        double p = exp(sr[kk - t0] - m_new);
        const double *vk = v + (size_t)kk * d_v;
        l[r] += p;
        for (int c = 0; c < d_v; ++c) ar[c] += p * vk[c];
      }
      m[r] = m_new;
    }
  }

  /* O = acc / l and LSE = m + ln l. A row with nothing accumulated gives O = 0, LSE = -inf. */
  for (int r = 0; r < n_rows; ++r) {
    double *orow = o + (size_t)r * d_v;
    const double *ar = acc + (size_t)r * d_v;
    if (l[r] > 0.0) {
      for (int c = 0; c < d_v; ++c) orow[c] = ar[c] / l[r];
      lse[r] = m[r] + log(l[r]);
    } else {
      for (int c = 0; c < d_v; ++c) orow[c] = 0.0;
      lse[r] = -INFINITY;
    }
    if (row_max) row_max[r] = m[r];
    if (row_sum) row_sum[r] = l[r];
  }
  free(m); free(l); free(mt); free(acc); free(s);
  return status;
}

/*
 * Merge partial results of disjoint key ranges by their log-sum-exp ([HG]: L = m + log l is
 * the log of the softmax denominator, so exp(L_s) is split s's denominator):
 *   M = max_s L_s,  w_s = exp(L_s - M),  O = sum_s w_s O_s / sum_s w_s,  L = M + ln sum_s w_s.
 * o_parts: n_splits x n_rows x d_v, lse_parts: n_splits x n_rows.
 */
int oracle_combine(int n_splits, int n_rows, int d_v, const double *o_parts,
                   const double *lse_parts, double *o, double *lse) {
  if (n_splits <= 0 || n_rows < 0 || d_v <= 0) return ORACLE_BAD_ARG;
  for (int r = 0; r < n_rows; ++r) {
    double mx = -INFINITY;
    for (int sp = 0; sp < n_splits; ++sp) {
      double x = lse_parts[(size_t)sp * n_rows + r];
      if (x > mx) mx = x;
    }
    double *orow = o + (size_t)r * d_v;
    for (int c = 0; c < d_v; ++c) orow[c] = 0.0;
    if (mx == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double wsum = 0.0;
    for (int sp = 0; sp < n_splits; ++sp) {
      double x = lse_parts[(size_t)sp * n_rows + r];
      if (x == -INFINITY) continue;
      double w = exp(x - mx);
      const double *op = o_parts + ((size_t)sp * n_rows + r) * d_v;
      wsum += w;
      for (int c = 0; c < d_v; ++c) orow[c] += w * op[c];
    }
    for (int c = 0; c < d_v; ++c) orow[c] /= wsum;
    lse[r] = mx + log(wsum);
  }
  return ORACLE_OK;
}

/* One independent unit of work for the batch driver: a block of rows against a key range. */
typedef struct {
  int n_rows;
  const double *q;
  const double *k;
  const double *v;
  const int *row_first; /* may be NULL */
  const int *row_keys;
  int k_begin, k_end;
  double *o;
  double *lse;
  unsigned char *tile_status; /* may be NULL */
  double *tile_margin;        /* may be NULL */
  int max_tiles;
  const unsigned char *forced; /* may be NULL: decisions to impose (see oracle_blasst_rows) */
  long long visited, skipped; /* outputs */
  int status;                 /* output */
} oracle_unit;

/*
 * Run independent units, one per OpenMP iteration. Units share nothing they write, so this is
 * the same as calling oracle_blasst_rows on each unit in turn. n_threads <= 0 keeps the OpenMP
 * default.
 */
int oracle_blasst_batch(int n_units, oracle_unit *units, int d_qk, int d_v, int block_c,
                        double scale, double lambda, int n_threads) {
  int worst = ORACLE_OK;
  int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int u = 0; u < n_units; ++u) {
    oracle_unit *un = &units[u];
    un->visited = 0;
    un->skipped = 0;
    un->status = oracle_blasst_rows(un->n_rows, d_qk, d_v, un->q, un->k, un->v, un->row_first,
                                    un->row_keys,
                                    un->k_begin, un->k_end, block_c, scale, lambda, un->o,
                                    un->lse, NULL, NULL, &un->visited, &un->skipped,
                                    un->tile_status, un->tile_margin, un->max_tiles,
                                    un->forced);
  }
  for (int u = 0; u < n_units; ++u)
    if (units[u].status != ORACLE_OK) worst = units[u].status;
  return worst;
}

/* Same driver for the dense definition (one unit = a block of rows against keys [0, k_end)). */
int oracle_dense_batch(int n_units, oracle_unit *units, int d_qk, int d_v, double scale,
                       int n_threads) {
  int worst = ORACLE_OK;
  int nt = n_threads > 0 ? n_threads : omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
  for (int u = 0; u < n_units; ++u) {
    oracle_unit *un = &units[u];
    un->status = oracle_dense_rows(un->n_rows, un->k_end, d_qk, d_v, un->q, un->k, un->v,
                                   un->row_first, un->row_keys, scale, un->o, un->lse);
  }
  for (int u = 0; u < n_units; ++u)
    if (units[u].status != ORACLE_OK) worst = units[u].status;
  return worst;
}

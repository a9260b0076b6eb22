/*
 * blasst.h -- C ABI of the BLASST skip-softmax attention forward pass for AMD Instinct MI355X
 * (gfx950).
 *
 * The method (cited by page title and section):
 *   - "Skip-Softmax" (vLLM-Omni feature design page), "Algorithm": FlashAttention's streaming
 *     pass over key tiles keeps a running max m, sum l and numerator O per query row; after a
 *     tile's scores are computed, the tile's softmax and its P.V product are skipped when
 *     exp(tile_max[i] - running_max[i]) < lambda for every query row i of the tile, which the
 *     kernel evaluates in log space as tile_max - running_max < ln(lambda).
 *   - same page, "From configuration to the kernel threshold": lambda = threshold, or
 *     threshold_scale_factor / max_kv_len, or a * exp(b * target_sparsity) / max_kv_len.
 *   - "BLASST: Dynamic BLocked Attention Sparsity via Softmax Thresholding" (MLSys 2026 talk
 *     notes), kernel design: prefill skips the softmax and the second matmul; decode also skips
 *     loading the value tile from memory, issuing value loads only after the test.
 *   - "The Hitchhiker's Guide -- Phase 08", Section 1: attention = softmax(QK^T / sqrt(d)) V,
 *     the online-softmax recurrence, tiling into B_r query rows x B_c keys visited in ascending
 *     key order, and the log-sum-exp output L = m + log(l).
 *
 * Conventions shared by every entry point:
 *   - Device pointers are HIP device memory owned by the caller; the library allocates nothing
 *     and keeps no state between calls. Launches are asynchronous on `stream` (a hipStream_t;
 *     NULL = the null stream). Kernel faults surface at the caller's next synchronisation.
 *   - A call issues nothing but kernel launches on `stream` (no allocation, memset, copy or
 *     host synchronisation), so it may be captured into a HIP graph; a replay reads the buffers'
 *     contents at replay time and, like an eager call, adds to `counters`.
 *   - Argument checks happen on the host before any launch; a failed check launches nothing and
 *     returns BLASST_ERR_INVALID_ARG or BLASST_ERR_UNSUPPORTED. A failed launch returns
 *     BLASST_ERR_HIP.
 *   - Strides are in elements, the last (feature) dimension is contiguous, base pointers are
 *     16-byte aligned and every stride is a multiple of 8 elements (bf16) or 4 elements (fp32).
 *   - lambda must be finite and >= 0. Values above 1 are treated as 1 (the test's left side lies
 *     in (0, 1], so lambda = 1 already skips every tile that holds no new row maximum); lambda = 0
 *     skips nothing and computes dense attention.
 *   - Optional observation outputs (counters, per-tile status and margin) may be NULL.
 *     `counters` is device memory of two uint64: visited tiles and skipped tiles, incremented
 *     atomically (the caller zeroes it). `tile_status` holds one byte per (unit, tile):
 *     0 kept, 1 skipped, 2 not visited. `tile_margin` holds the tile's margin
 *     max over rows of (tile_max - running_max) in natural-log units (-inf if not visited).
 */
#ifndef BLASST_H
#define BLASST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum blasst_status {
  BLASST_OK = 0,
  BLASST_ERR_INVALID_ARG = 1,    /* NULL pointer, bad shape, NaN/negative lambda, bad stride */
  BLASST_ERR_UNSUPPORTED = 2,    /* valid but not implemented: head dim, dtype, tile shape */
  BLASST_ERR_NO_CALIBRATION = 3, /* target sparsity requested without coefficients a, b */
  BLASST_ERR_CONFLICT = 4,       /* both a threshold and a target sparsity given */
  BLASST_ERR_HIP = 5,            /* a HIP runtime call failed (launch) */
  BLASST_ERR_WORKSPACE = 6       /* workspace missing or smaller than required */
} blasst_status;

/* Returns a static, human-readable name for a status code. */
const char *blasst_status_string(blasst_status status);

/* ------------------------------------------------------------------------------------------
 * Threshold resolution ("Skip-Softmax" page, "From configuration to the kernel threshold";
 * BLASST notes, threshold calibration, Eq. 3: lambda = a / L).
 *
 *   BLASST_DENSE           lambda = 0 (no tile is skipped).
 *   BLASST_THRESHOLD       lambda = threshold (independent of the sequence length).
 *   BLASST_SCALE_FACTOR    lambda = scale_factor / max_kv_len (the factor the kernel of the
 *                          page takes; Eq. 3's a / L).
 *   BLASST_TARGET_SPARSITY lambda = a * exp(b * target_sparsity) / max_kv_len, with a and b the
 *                          calibration coefficients (has_calibration != 0).
 *
 * Errors: spec or lambda_out NULL, max_kv_len <= 0 (modes that divide by it), NaN / infinite /
 * negative threshold or scale factor, target_sparsity outside [0, 1] or NaN, a non-finite
 * result -> BLASST_ERR_INVALID_ARG. A target sparsity without calibration ->
 * BLASST_ERR_NO_CALIBRATION (the page's startup rule points the user to `threshold` instead; a
 * layer whose coefficients are missing runs dense, which the caller does by using lambda = 0).
 * BLASST_ERR_CONFLICT if a threshold-type field and a target are both set (threshold > 0 in
 * BLASST_TARGET_SPARSITY mode). The result is not clamped here; the kernels clamp to [0, 1].
 * ------------------------------------------------------------------------------------------ */
typedef enum blasst_mode {
  BLASST_DENSE = 0,
  BLASST_THRESHOLD = 1,
  BLASST_SCALE_FACTOR = 2,
  BLASST_TARGET_SPARSITY = 3
} blasst_mode;

typedef struct blasst_lambda_spec {
  blasst_mode mode;
  double threshold;       /* BLASST_THRESHOLD */
  double scale_factor;    /* BLASST_SCALE_FACTOR */
  double target_sparsity; /* BLASST_TARGET_SPARSITY, in [0, 1] */
  int32_t has_calibration;
  double a, b;            /* calibration: lambda * L = a * exp(b * S) */
} blasst_lambda_spec;

blasst_status blasst_resolve_lambda(const blasst_lambda_spec *spec, int64_t max_kv_len,
                                    double *lambda_out);

/* ------------------------------------------------------------------------------------------
 * Calibration (BLASST notes, threshold calibration, Algorithm 2 steps 1-3 and Eq. 3).
 *
 * blasst_sparsity_curve: step 1, many candidate thresholds from one pass. A tile's margin
 * (tile_max - running_max, natural log, as the attention calls write to tile_margin) does not
 * depend on lambda -- the running max advances whether or not a tile is skipped -- so the tiles a
 * call with threshold lambda skips are exactly the visited tiles with margin < ln(min(lambda, 1)).
 *   tile_margin, tile_status: host arrays of n_tiles entries as one attention call wrote them
 *     (status 0 or 1 = visited, 2 = not visited; any other status is an error).
 *   lambdas: n_lambdas finite non-negative candidates.
 *   sparsity (out, n_lambdas): skipped / visited for each candidate (0 when nothing was visited).
 *   visited (out, may be NULL): the number of visited tiles.
 * Errors: NULL arrays with a positive count, n_tiles or n_lambdas < 0, a bad lambda, an unknown
 * status -> BLASST_ERR_INVALID_ARG. Host memory only; no device call.
 *
 * blasst_fit_calibration: step 3, the exponential model lambda * L = a * exp(b * S) fitted by
 * least squares on ln(lambda * L) = ln a + b S over n observations (seq_len L > 0, lambda > 0,
 * sparsity S finite). The (a, b) it returns feed BLASST_TARGET_SPARSITY.
 * Errors: NULL pointers, n < 2, a non-positive or non-finite L or lambda, non-finite S, or all S
 * equal -> BLASST_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------------------------ */
blasst_status blasst_sparsity_curve(const float *tile_margin, const uint8_t *tile_status,
                                    int64_t n_tiles, const double *lambdas, int32_t n_lambdas,
                                    double *sparsity, int64_t *visited);

blasst_status blasst_fit_calibration(const double *seq_len, const double *lambda,
                                     const double *sparsity, int32_t n, double *a, double *b);

/* ------------------------------------------------------------------------------------------
 * Timestep gate ("Skip-Softmax" page, "Timestep gating"): whether skipping is active on a
 * diffusion step with normalised timestep t in [0, 1] (decreasing over the run).
 *   disabled_until_timestep == 0: the gate is off, skipping is active on every step (t unused).
 *   otherwise: skipping is active iff the pipeline publishes t and t <= the cutoff.
 * has_t = 0 (t not published) with a positive cutoff: stays dense (the caller logs once).
 * Writes 1 (skip active) or 0 (dense) to *active. Errors: NULL active, cutoff NaN / negative,
 * has_t with NaN t -> BLASST_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------------------------ */
blasst_status blasst_timestep_gate(double disabled_until_timestep, int32_t has_t, double t,
                                   int32_t *active);

typedef enum blasst_dtype { BLASST_F32 = 0, BLASST_BF16 = 1 } blasst_dtype;

/* ------------------------------------------------------------------------------------------
 * Prefill / full self-attention forward pass, MHA or GQA, causal or not.
 *
 *   q [batch, len_q, heads_q, head_dim]   k, v [batch, len_kv, heads_kv, head_dim]
 *   o [batch, len_q, heads_q, head_dim]   lse (optional, fp32) [batch, heads_q, len_q] contiguous
 * (any strides that meet the conventions above; dims given as [batch, seq, head]).
 *
 * Query head h uses KV head h / (heads_q / heads_kv). With causal != 0 (requires len_q ==
 * len_kv) query position i sees keys 0..i. Work unit = (batch, head, block of block_r query
 * positions); its key tiles of block_c keys are visited in ascending order; a tile that no row
 * of the block can see is not visited. The skip test is taken per (unit, tile) over all block_r
 * rows; a row that sees no key of the tile votes "skip".
 *
 * Sliding window (window > 0, causal only; the BLASST talk notes' Q&A names windowed attention
 * as structured sparsity the method carries over to): query position i sees keys
 * max(0, i - window + 1) .. i. Key tiles before every row of a block's window are not visited,
 * and keys outside a row's window score -inf. window 0 = no window.
 *
 * Supported: dtype BLASST_BF16 or BLASST_F32, head_dim 64 or 128, block_r 32, 64 or 128
 * (default 128 for bf16, 64 for fp32), block_c 64 (blasst_prefill_tiles resolves defaults). softmax_scale 0 means 1/sqrt(head_dim). o is written in dtype; lse in natural
 * log units. Observation outputs: tile_status / tile_margin are
 * [batch, heads_q, ceil(len_q / block_r), ceil(len_kv / block_c)].
 * ------------------------------------------------------------------------------------------ */
typedef struct blasst_prefill_args {
  blasst_dtype dtype;
  int32_t batch, heads_q, heads_kv, len_q, len_kv, head_dim;
  int32_t causal;
  const void *q, *k, *v;
  void *o;
  int64_t q_stride[3], k_stride[3], v_stride[3], o_stride[3];
  float softmax_scale;
  double lambda;
  float *lse;
  unsigned long long *counters;
  uint8_t *tile_status;
  float *tile_margin;
  int32_t block_r, block_c; /* 0 = default */
  int32_t window;           /* sliding window in keys (causal only); 0 = none */
} blasst_prefill_args;

blasst_status blasst_attn_prefill(const blasst_prefill_args *args, void *stream);

/* The (block_r, block_c) a prefill call with these arguments uses (resolves the defaults);
 * BLASST_ERR_UNSUPPORTED if the combination has no kernel. */
blasst_status blasst_prefill_tiles(const blasst_prefill_args *args, int32_t *block_r,
                                   int32_t *block_c);

/* ------------------------------------------------------------------------------------------
 * Decode: one query token per sequence against its KV cache (GQA / MQA, or MLA-shaped where V
 * is the first head_dim_v columns of K and v may alias k).
 *
 *   q [batch, heads_q, head_dim_qk]      o [batch, heads_q, head_dim_v]  (strides: batch, head)
 *   k [batch, max_kv_len, heads_kv, head_dim_qk], v [batch, max_kv_len, heads_kv, head_dim_v]
 *     (strides: batch, seq, head)
 *   kv_len (optional, device int32 [batch]): sequence b uses keys [0, kv_len[b]); NULL = all
 *     max_kv_len. Each kv_len[b] must lie in [0, max_kv_len]. A sequence of length 0 gets
 *     o = 0 and lse = -inf.
 *   lse (optional, fp32) [batch, heads_q] contiguous, natural log.
 *
 * Work unit = (batch, KV head g, block of block_r query heads among the heads_q / heads_kv heads
 * that share g); the rows of a tile are those query heads. With num_splits S > 1 the key tiles
 * are cut into S runs of ceil(ceil(max_kv_len / block_c) / S) tiles; each run restarts the
 * running max, writes a partial (o, lse) to the workspace and a merge kernel combines them by
 * log-sum-exp. num_splits 0 = chosen by the library (blasst_decode_plan reports the choice).
 *
 * Sliding window (window > 0): the query of sequence b (at position kv_len[b] - 1) sees keys
 * max(0, kv_len[b] - window) .. kv_len[b] - 1. The splits then cut the at most
 * ceil(window / block_c) + 1 tiles a window touches, starting at the tile that holds the
 * sequence's first visible key; tiles outside every split are not visited. window 0 = none.
 *
 * Value loads are issued only for kept tiles. With v == k and head_dim_v < head_dim_qk (MLA
 * shape) the value tile is read from the key tile already on chip, so skipping saves compute.
 *
 * Supported: BLASST_BF16; GQA kernel: head_dim_qk == head_dim_v == 128 (or 64), block_c 64,
 * block_r <= 16; MLA kernels: head_dim_qk 576, head_dim_v 512, heads_kv 1, v == k, block_c 64,
 * block_r 64 or 128 (0 = 128 when heads_q > 64, else 64; a block larger than heads_q is cut to
 * heads_q). With block_r 128 one unit covers up to 128 heads and each K tile is read once for
 * all of them. tile_status / tile_margin:
 * [batch, heads_kv, ceil(G / block_r), ceil(max_kv_len / block_c)], G = heads_q / heads_kv.
 *
 * Paged KV cache ("The Hitchhiker's Guide -- Phase 08", paged attention: a block table maps a
 * sequence position to a physical block). With block_table != NULL, k and v point at page pools
 * addressed [page, row, head, dim] by their strides (k_stride[0] is the page stride, k_stride[1]
 * the row stride); key t of sequence b is row t % page_size of page
 * block_table[b * pages_per_seq + t / page_size]. page_size: a power of two in [1, 4096];
 * pages_per_seq * page_size >= max_kv_len. The table is device int32 memory owned by the caller;
 * its entries for the keys a sequence uses must name pages inside the pools (they are not
 * checked on the host: an entry out of range reads outside the pool). Results are bit-identical
 * to a contiguous cache holding the same keys. block_table == NULL: contiguous per sequence
 * (page_size and pages_per_seq ignored).
 * ------------------------------------------------------------------------------------------ */
typedef struct blasst_decode_args {
  blasst_dtype dtype;
  int32_t batch, heads_q, heads_kv, max_kv_len, head_dim_qk, head_dim_v;
  const void *q, *k, *v;
  void *o;
  int64_t q_stride[2], k_stride[3], v_stride[3], o_stride[2];
  const int32_t *kv_len;
  float softmax_scale;
  double lambda;
  float *lse;
  unsigned long long *counters;
  uint8_t *tile_status;
  float *tile_margin;
  int32_t block_r, block_c, num_splits; /* 0 = default / automatic */
  const int32_t *block_table;           /* optional paged cache: device [batch, pages_per_seq] */
  int32_t page_size, pages_per_seq;
  int32_t window;                       /* sliding window in keys; 0 = none */
} blasst_decode_args;

/* Resolved launch plan of a decode call: tile shape and split count. */
blasst_status blasst_decode_plan(const blasst_decode_args *args, int32_t *block_r,
                                 int32_t *block_c, int32_t *num_splits);

/* Bytes of device workspace a decode call needs (0 when it runs unsplit). */
size_t blasst_decode_workspace_size(const blasst_decode_args *args);

/* workspace: device memory of at least blasst_decode_workspace_size(args) bytes (may be NULL
 * when that is 0), 256-byte aligned, not used by another call in flight. */
blasst_status blasst_attn_decode(const blasst_decode_args *args, void *workspace,
                                 size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------------------------
 * Decode without any allocation, for callers that cannot call hipMalloc: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. The same call as
 * blasst_attn_decode (same kernels, same results bit for bit), but the split partials live in a
 * scratch array of BLASST_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends; the caller passes inputs and outputs only.
 *
 *   - The stream must belong to the current HIP device (the scratch array used is that device's).
 *     The first call on a device looks up the array's device address; no call allocates or
 *     frees memory, and no call issues a memset or copy.
 *   - A call whose blasst_decode_workspace_size exceeds BLASST_NOALLOC_SCRATCH_BYTES returns
 *     BLASST_ERR_WORKSPACE before touching the device (ask for fewer splits, or use
 *     blasst_attn_decode with a workspace). Other errors as for blasst_attn_decode.
 *   - Every call on one GPU shares that GPU's array and leaves its partials there: calls that
 *     overlap in time on one GPU (two streams, two host threads) race and give wrong results.
 *     Calls ordered on one stream are safe.
 * ------------------------------------------------------------------------------------------ */
#define BLASST_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u) /* 128 MiB per GPU */
blasst_status blasst_attn_decode_noalloc(const blasst_decode_args *args, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* BLASST_H */

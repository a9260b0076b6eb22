// api.cpp -- host side of the C ABI in include/blasst.h: argument checks, threshold resolution,
// launch planning and dispatch to the HIP kernels. Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "blasst.h"
#include "internal.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;

bool finite_nonneg(double x) { return isfinite(x) && x >= 0.0; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Base-2 threshold the kernels compare against: log2(min(lambda, 1)), -inf for lambda == 0.
float tau_log2(double lambda) {
  const double lam = lambda > 1.0 ? 1.0 : lambda;
  return lam > 0.0 ? (float)log2(lam) : -INFINITY;
}

float scale_log2(float softmax_scale, int head_dim) {
  const double s = softmax_scale > 0.f ? (double)softmax_scale : 1.0 / sqrt((double)head_dim);
  return (float)(s * kLog2e);
}

bool strides_ok(const int64_t *st, int n, int64_t mult) {
  for (int i = 0; i < n; ++i)
    if (st[i] < 0 || st[i] % mult != 0) return false;
  return true;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// The integer a caller stored in an enum field of an argument struct. Callers in C (or through
// an FFI) may store any int there; reading such a value through the C++ enum type is undefined,
// so the bytes are read as an int and compared against the named values.
template <typename E>
int32_t enum_int(const E &e) {
  static_assert(sizeof(E) == sizeof(int32_t), "enum fields are 32-bit");
  int32_t v;
  memcpy(&v, &e, sizeof v);
  return v;
}

}  // namespace

extern "C" {

const char *blasst_status_string(blasst_status status) {
  switch (status) {
    case BLASST_OK: return "BLASST_OK";
    case BLASST_ERR_INVALID_ARG: return "BLASST_ERR_INVALID_ARG";
    case BLASST_ERR_UNSUPPORTED: return "BLASST_ERR_UNSUPPORTED";
    case BLASST_ERR_NO_CALIBRATION: return "BLASST_ERR_NO_CALIBRATION";
    case BLASST_ERR_CONFLICT: return "BLASST_ERR_CONFLICT";
    case BLASST_ERR_HIP: return "BLASST_ERR_HIP";
    case BLASST_ERR_WORKSPACE: return "BLASST_ERR_WORKSPACE";
  }
  return "BLASST_UNKNOWN_STATUS";
}

// "Skip-Softmax" page, "From configuration to the kernel threshold": the kernel receives
// threshold_scale_factor and divides it by the call's max_kv_len; a threshold t is passed as
// t * max_kv_len (so lambda = t); a target sparsity s is passed as a * exp(b * s).
blasst_status blasst_resolve_lambda(const blasst_lambda_spec *spec, int64_t max_kv_len,
                                    double *lambda_out) {
  if (!spec || !lambda_out) return BLASST_ERR_INVALID_ARG;
  switch (enum_int(spec->mode)) {
    case BLASST_DENSE:
      *lambda_out = 0.0;
      return BLASST_OK;
    case BLASST_THRESHOLD:
      if (!finite_nonneg(spec->threshold)) return BLASST_ERR_INVALID_ARG;
      *lambda_out = spec->threshold;
      return BLASST_OK;
    case BLASST_SCALE_FACTOR: {
      if (!finite_nonneg(spec->scale_factor) || max_kv_len <= 0) return BLASST_ERR_INVALID_ARG;
      const double lam = spec->scale_factor / (double)max_kv_len;
      if (!isfinite(lam)) return BLASST_ERR_INVALID_ARG;
      *lambda_out = lam;
      return BLASST_OK;
    }
    case BLASST_TARGET_SPARSITY: {
      if (spec->threshold > 0.0 || spec->scale_factor > 0.0) return BLASST_ERR_CONFLICT;
      const double s = spec->target_sparsity;
      if (!(s >= 0.0 && s <= 1.0) || max_kv_len <= 0) return BLASST_ERR_INVALID_ARG;
      if (!spec->has_calibration) return BLASST_ERR_NO_CALIBRATION;
      if (!isfinite(spec->a) || !isfinite(spec->b) || spec->a < 0.0) return BLASST_ERR_INVALID_ARG;
      const double lam = spec->a * exp(spec->b * s) / (double)max_kv_len;
      if (!finite_nonneg(lam)) return BLASST_ERR_INVALID_ARG;
      *lambda_out = lam;
      return BLASST_OK;
    }
  }
  return BLASST_ERR_INVALID_ARG;
}

// BLASST notes, threshold calibration, Algorithm 2 step 1: the skip fraction at many thresholds
// from the margins of one call. A skipped tile is a visited tile whose margin is below
// ln(min(lambda, 1)); lambda = 0 (ln 0 = -inf) skips nothing.
blasst_status blasst_sparsity_curve(const float *tile_margin, const uint8_t *tile_status,
                                    int64_t n_tiles, const double *lambdas, int32_t n_lambdas,
                                    double *sparsity, int64_t *visited) {
  if (n_tiles < 0 || n_lambdas < 0) return BLASST_ERR_INVALID_ARG;
  if (n_tiles > 0 && (!tile_margin || !tile_status)) return BLASST_ERR_INVALID_ARG;
  if (n_lambdas > 0 && (!lambdas || !sparsity)) return BLASST_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n_lambdas; ++i)
    if (!finite_nonneg(lambdas[i])) return BLASST_ERR_INVALID_ARG;
  int64_t n_vis = 0;
  for (int64_t t = 0; t < n_tiles; ++t) {
    if (tile_status[t] > 2) return BLASST_ERR_INVALID_ARG;
    n_vis += tile_status[t] != 2;
  }
  for (int32_t i = 0; i < n_lambdas; ++i) {
    const double lam = lambdas[i] < 1.0 ? lambdas[i] : 1.0;
    const double tau = lam > 0.0 ? log(lam) : -INFINITY;
    int64_t n_skip = 0;
    for (int64_t t = 0; t < n_tiles; ++t)
      n_skip += tile_status[t] != 2 && (double)tile_margin[t] < tau;
    sparsity[i] = n_vis > 0 ? (double)n_skip / (double)n_vis : 0.0;
  }
  if (visited) *visited = n_vis;
  return BLASST_OK;
}

// BLASST notes, threshold calibration, Algorithm 2 step 3 (model lambda * L = a * exp(b * S)):
// ordinary least squares of y = ln(lambda * L) on S.
blasst_status blasst_fit_calibration(const double *seq_len, const double *lambda,
                                     const double *sparsity, int32_t n, double *a, double *b) {
  if (!seq_len || !lambda || !sparsity || !a || !b || n < 2) return BLASST_ERR_INVALID_ARG;
  double ms = 0.0, my = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    if (!(seq_len[i] > 0.0) || !isfinite(seq_len[i]) || !(lambda[i] > 0.0) ||
        !isfinite(lambda[i]) || !isfinite(sparsity[i]))
      return BLASST_ERR_INVALID_ARG;
    ms += sparsity[i];
    my += log(lambda[i] * seq_len[i]);
  }
  ms /= n;
  my /= n;
  double sxx = 0.0, sxy = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    const double dx = sparsity[i] - ms;
    sxx += dx * dx;
    sxy += dx * (log(lambda[i] * seq_len[i]) - my);
  }
  if (!(sxx > 0.0)) return BLASST_ERR_INVALID_ARG;
  *b = sxy / sxx;
  *a = exp(my - *b * ms);
  if (!isfinite(*a) || !isfinite(*b)) return BLASST_ERR_INVALID_ARG;
  return BLASST_OK;
}

// "Skip-Softmax" page, "Timestep gating": dense while t is above the cutoff; cutoff 0 is the
// "gate off" sentinel; without a published t a positive cutoff keeps the call dense.
blasst_status blasst_timestep_gate(double disabled_until_timestep, int32_t has_t, double t,
                                   int32_t *active) {
  if (!active || !(disabled_until_timestep >= 0.0) || !isfinite(disabled_until_timestep))
    return BLASST_ERR_INVALID_ARG;
  if (disabled_until_timestep == 0.0) {
    *active = 1;
    return BLASST_OK;
  }
  if (!has_t) {
    *active = 0;
    return BLASST_OK;
  }
  if (isnan(t)) return BLASST_ERR_INVALID_ARG;
  *active = t <= disabled_until_timestep ? 1 : 0;
  return BLASST_OK;
}

// ------------------------------------------------------------------------------------------
// Prefill
// ------------------------------------------------------------------------------------------
blasst_status blasst_prefill_tiles(const blasst_prefill_args *a, int32_t *block_r,
                                   int32_t *block_c) {
  if (!a || !block_r || !block_c) return BLASST_ERR_INVALID_ARG;
  const int32_t dtype = enum_int(a->dtype);
  if (dtype != BLASST_BF16 && dtype != BLASST_F32) return BLASST_ERR_UNSUPPORTED;
  const int br = a->block_r ? a->block_r : (dtype == BLASST_BF16 ? 128 : 64);
  const int bc = a->block_c ? a->block_c : blasst::kBlockC;
  if (br != 32 && br != 64 && br != 128) return BLASST_ERR_UNSUPPORTED;
  if (bc != blasst::kBlockC) return BLASST_ERR_UNSUPPORTED;
  *block_r = br;
  *block_c = bc;
  return BLASST_OK;
}

blasst_status blasst_attn_prefill(const blasst_prefill_args *a, void *stream) {
  if (!a) return BLASST_ERR_INVALID_ARG;
  const int32_t dtype = enum_int(a->dtype);
  if (dtype != BLASST_BF16 && dtype != BLASST_F32) return BLASST_ERR_UNSUPPORTED;
  if (a->batch < 0 || a->len_q < 0 || a->len_kv < 0 || a->heads_q <= 0 || a->heads_kv <= 0)
    return BLASST_ERR_INVALID_ARG;
  if (a->heads_q % a->heads_kv != 0) return BLASST_ERR_INVALID_ARG;
  if (a->causal && a->len_q != a->len_kv) return BLASST_ERR_INVALID_ARG;
  if (a->window < 0) return BLASST_ERR_INVALID_ARG;
  if (a->window > 0 && !a->causal) return BLASST_ERR_UNSUPPORTED;
  if (!finite_nonneg(a->lambda)) return BLASST_ERR_INVALID_ARG;
  if (!(a->softmax_scale >= 0.f) || !isfinite(a->softmax_scale)) return BLASST_ERR_INVALID_ARG;
  if (a->head_dim != 64 && a->head_dim != 128) return BLASST_ERR_UNSUPPORTED;
  int32_t br, bc;
  blasst_status st = blasst_prefill_tiles(a, &br, &bc);
  if (st != BLASST_OK) return st;
  if (a->batch == 0 || a->len_q == 0) return BLASST_OK;  // nothing to compute
  if (a->len_kv == 0) return BLASST_ERR_INVALID_ARG;      // rows with no key at all
  if (!a->q || !a->k || !a->v || !a->o) return BLASST_ERR_INVALID_ARG;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return BLASST_ERR_INVALID_ARG;
  const int64_t mult = dtype == BLASST_BF16 ? 8 : 4;
  if (!strides_ok(a->q_stride, 3, mult) || !strides_ok(a->k_stride, 3, mult) ||
      !strides_ok(a->v_stride, 3, mult) || !strides_ok(a->o_stride, 3, mult))
    return BLASST_ERR_INVALID_ARG;
  const int n_qb = ceil_div(a->len_q, br);
  if (a->heads_q > 65535 || a->batch > 65535) return BLASST_ERR_UNSUPPORTED;

  blasst::PrefillParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o;
  p.q_sb = a->q_stride[0]; p.q_ss = a->q_stride[1]; p.q_sh = a->q_stride[2];
  p.k_sb = a->k_stride[0]; p.k_ss = a->k_stride[1]; p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0]; p.v_ss = a->v_stride[1]; p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0]; p.o_ss = a->o_stride[1]; p.o_sh = a->o_stride[2];
  p.B = a->batch; p.Hq = a->heads_q; p.Hkv = a->heads_kv; p.Lq = a->len_q; p.Lkv = a->len_kv;
  p.causal = a->causal ? 1 : 0;
  p.n_qblocks = n_qb;
  p.n_kvtiles = ceil_div(a->len_kv, bc);
  p.scale_log2 = scale_log2(a->softmax_scale, a->head_dim);
  p.tau_log2 = tau_log2(a->lambda);
  p.lse = a->lse;
  p.counters = a->counters;
  p.tile_status = a->tile_status;
  p.tile_margin = a->tile_margin;
  p.window = a->window;
  const hipError_t err =
      blasst::launch_prefill(p, dtype == BLASST_BF16 ? 1 : 0, a->head_dim, br,
                             (hipStream_t)stream);
  return err == hipSuccess ? BLASST_OK : BLASST_ERR_HIP;
}

// ------------------------------------------------------------------------------------------
// Decode
// ------------------------------------------------------------------------------------------
namespace {

enum DecodeKind { kNone = 0, kGqa = 1, kMla = 2 };

DecodeKind decode_kind(const blasst_decode_args *a) {
  if (enum_int(a->dtype) != BLASST_BF16) return kNone;
  if (a->head_dim_qk == a->head_dim_v && (a->head_dim_qk == 128 || a->head_dim_qk == 64))
    return kGqa;
  if (a->head_dim_qk == 576 && a->head_dim_v == 512 && a->heads_kv == 1 && a->v == a->k)
    return kMla;
  return kNone;
}

// Split count chosen by the library: at least `target` work units (every CU about two of them
// by default), but at least 8 tiles per split.
int auto_splits(int units, int n_tiles, int target = 2 * 256) {
  if (units >= target || n_tiles <= 8) return 1;
  int s = ceil_div(target, units);
  const int max_s = n_tiles / 8 > 0 ? n_tiles / 8 : 1;
  if (s > max_s) s = max_s;
  if (s > 64) s = 64;
  return s < 1 ? 1 : s;
}

// Tiles the splits of one sequence divide: all of max_kv_len, or with a sliding window the at
// most ceil(window / B_c) + 1 tiles a window of that many keys can touch.
int split_span(const blasst_decode_args *a, int bc) {
  const int n_tiles = ceil_div(a->max_kv_len, bc);
  if (a->window <= 0) return n_tiles;
  const int w = ceil_div(a->window, bc) + 1;
  return w < n_tiles ? w : n_tiles;
}

}  // namespace

blasst_status blasst_decode_plan(const blasst_decode_args *a, int32_t *block_r, int32_t *block_c,
                                 int32_t *num_splits) {
  if (!a || !block_r || !block_c || !num_splits) return BLASST_ERR_INVALID_ARG;
  if (a->heads_q <= 0 || a->heads_kv <= 0 || a->heads_q % a->heads_kv != 0 || a->batch < 0 ||
      a->max_kv_len < 0 || a->window < 0)
    return BLASST_ERR_INVALID_ARG;
  const DecodeKind kind = decode_kind(a);
  if (kind == kNone) return BLASST_ERR_UNSUPPORTED;
  const int group = a->heads_q / a->heads_kv;
  const int bc = a->block_c ? a->block_c : blasst::kBlockC;
  if (bc != blasst::kBlockC) return BLASST_ERR_UNSUPPORTED;
  int br;
  if (kind == kGqa) {
    br = a->block_r ? a->block_r : (group < 16 ? group : 16);
    if (br < 1 || br > 16) return BLASST_ERR_UNSUPPORTED;
  } else {
    // MLA: a unit of up to 128 heads (one workgroup fills a CU) when the group has more than 64,
    // else the 64-head kernel.
    br = a->block_r ? a->block_r : (group > 64 ? 128 : 64);
    if (br != 64 && br != 128) return BLASST_ERR_UNSUPPORTED;
  }
  const bool wide_mla = kind == kMla && br > 64 && group > 64;
  if (br > group) br = group;
  int s = a->num_splits;
  if (s < 0) return BLASST_ERR_INVALID_ARG;
  if (s == 0) {
    const int units = a->batch * a->heads_kv * ceil_div(group, br);
    s = auto_splits(units > 0 ? units : 1, split_span(a, bc), wide_mla ? 256 : 2 * 256);
  }
  if (s > 256) return BLASST_ERR_UNSUPPORTED;
  *block_r = br;
  *block_c = bc;
  *num_splits = s;
  return BLASST_OK;
}

size_t blasst_decode_workspace_size(const blasst_decode_args *a) {
  int32_t br, bc, s;
  if (blasst_decode_plan(a, &br, &bc, &s) != BLASST_OK || s <= 1) return 0;
  const size_t rows = (size_t)a->batch * (size_t)a->heads_q * (size_t)s;
  const size_t o_bytes = rows * (size_t)a->head_dim_v * sizeof(float);
  const size_t l_bytes = rows * sizeof(float);
  return ((o_bytes + 255) / 256) * 256 + ((l_bytes + 255) / 256) * 256;
}

}  // extern "C"

namespace blasst {

blasst_status decode_check(const blasst_decode_args *a) {
  if (!a) return BLASST_ERR_INVALID_ARG;
  if (!finite_nonneg(a->lambda)) return BLASST_ERR_INVALID_ARG;
  if (!(a->softmax_scale >= 0.f) || !isfinite(a->softmax_scale)) return BLASST_ERR_INVALID_ARG;
  int32_t br, bc, s;
  return blasst_decode_plan(a, &br, &bc, &s);
}

blasst_status decode_with_workspace(const blasst_decode_args *a, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  if (!a) return BLASST_ERR_INVALID_ARG;
  if (!finite_nonneg(a->lambda)) return BLASST_ERR_INVALID_ARG;
  if (!(a->softmax_scale >= 0.f) || !isfinite(a->softmax_scale)) return BLASST_ERR_INVALID_ARG;
  int32_t br, bc, s;
  blasst_status st = blasst_decode_plan(a, &br, &bc, &s);
  if (st != BLASST_OK) return st;
  if (a->batch == 0) return BLASST_OK;
  if (!a->q || !a->k || !a->v || !a->o) return BLASST_ERR_INVALID_ARG;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return BLASST_ERR_INVALID_ARG;
  if (!strides_ok(a->q_stride, 2, 8) || !strides_ok(a->k_stride, 3, 8) ||
      !strides_ok(a->v_stride, 3, 8) || !strides_ok(a->o_stride, 2, 8))
    return BLASST_ERR_INVALID_ARG;
  if (a->batch > 65535 || a->heads_kv > 65535) return BLASST_ERR_UNSUPPORTED;
  int page_shift = 0;
  if (a->block_table) {
    // Paged cache: a power-of-two page size and enough pages per sequence for max_kv_len.
    if (a->page_size < 1 || a->page_size > 4096 || (a->page_size & (a->page_size - 1)) ||
        a->pages_per_seq < 1 ||
        (int64_t)a->pages_per_seq * a->page_size < (int64_t)a->max_kv_len)
      return BLASST_ERR_INVALID_ARG;
    while ((1 << page_shift) < a->page_size) ++page_shift;
  }
  const size_t need = blasst_decode_workspace_size(a);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255u)))
    return BLASST_ERR_WORKSPACE;

  const DecodeKind kind = decode_kind(a);
  blasst::DecodeParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->o;
  p.q_sb = a->q_stride[0]; p.q_sh = a->q_stride[1];
  p.k_sb = a->k_stride[0]; p.k_ss = a->k_stride[1]; p.k_sh = a->k_stride[2];
  p.v_sb = a->v_stride[0]; p.v_ss = a->v_stride[1]; p.v_sh = a->v_stride[2];
  p.o_sb = a->o_stride[0]; p.o_sh = a->o_stride[1];
  p.kv_len = a->kv_len;
  p.B = a->batch; p.Hq = a->heads_q; p.Hkv = a->heads_kv; p.max_kv_len = a->max_kv_len;
  p.group = a->heads_q / a->heads_kv;
  p.block_r = br;
  p.n_rblocks = ceil_div(p.group, br);
  p.n_tiles = ceil_div(a->max_kv_len, bc);
  p.num_splits = s;
  const int span = split_span(a, bc);
  p.tiles_per_split = span > 0 ? ceil_div(span, s) : 0;
  p.window = a->window;
  p.scale_log2 = scale_log2(a->softmax_scale, a->head_dim_qk);
  p.tau_log2 = tau_log2(a->lambda);
  p.lse = a->lse;
  p.counters = a->counters;
  p.tile_status = a->tile_status;
  p.tile_margin = a->tile_margin;
  p.block_table = a->block_table;
  p.page_shift = page_shift;
  p.pages_per_seq = a->block_table ? a->pages_per_seq : 0;
  if (s > 1) {
    const size_t rows = (size_t)a->batch * (size_t)a->heads_q * (size_t)s;
    const size_t o_bytes = ((rows * (size_t)a->head_dim_v * sizeof(float) + 255) / 256) * 256;
    p.o_part = (float *)workspace;
    p.lse_part = (float *)((char *)workspace + o_bytes);
  }
  hipError_t err;
  if (kind == kGqa) {
    err = blasst::launch_decode_gqa(p, a->head_dim_qk, (hipStream_t)stream);
  } else if (br > 64) {
    err = blasst::launch_decode_mla128(p, (hipStream_t)stream);
  } else {
    err = blasst::launch_decode_mla(p, (hipStream_t)stream);
  }
  if (err == hipSuccess && s > 1)
    err = blasst::launch_split_combine(p, a->head_dim_v, (hipStream_t)stream);
  return err == hipSuccess ? BLASST_OK : BLASST_ERR_HIP;
}

}  // namespace blasst

extern "C" blasst_status blasst_attn_decode(const blasst_decode_args *a, void *workspace,
                                            size_t workspace_bytes, void *stream) {
  return blasst::decode_with_workspace(a, workspace, workspace_bytes, stream);
}

// internal.h -- launch parameters shared by the host entry points and the HIP kernels.
// Not part of the public ABI (include/blasst.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "blasst.h"

namespace blasst {

// Key tile width of every kernel here (B_c).
constexpr int kBlockC = 64;

struct PrefillParams {
  const void *q, *k, *v;
  void *o;
  int64_t q_sb, q_ss, q_sh;  // strides in elements: batch, seq, head
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  int B, Hq, Hkv, Lq, Lkv;
  int causal;
  int n_qblocks, n_kvtiles;
  float scale_log2;  // softmax scale * log2(e): scores are kept in base-2 units
  float tau_log2;    // log2(min(lambda, 1)), -inf for lambda == 0
  float *lse;
  unsigned long long *counters;
  uint8_t *tile_status;
  float *tile_margin;
  int window;  // causal sliding window in keys (row i sees keys i - window + 1 .. i); 0 = none
};

// dtype: 0 fp32, 1 bf16. Returns hipSuccess or the launch error.
hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, int block_r,
                          hipStream_t stream);
// bf16, B_r = 128: the MFMA kernel with direct-to-LDS tile loads (prefill_mfma.hip).
hipError_t launch_prefill_mfma(const PrefillParams &p, int head_dim, hipStream_t stream);

struct DecodeParams {
  const void *q, *k, *v;
  void *o;
  int64_t q_sb, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_sh;
  const int32_t *kv_len;  // may be null: every sequence has max_kv_len keys
  int B, Hq, Hkv, max_kv_len;
  int group;           // Hq / Hkv
  int block_r;         // query heads per unit
  int n_rblocks;       // ceil(group / block_r)
  int num_splits;
  int tiles_per_split;
  int n_tiles;         // ceil(max_kv_len / B_c)
  float scale_log2;
  float tau_log2;
  float *lse;
  unsigned long long *counters;
  uint8_t *tile_status;
  float *tile_margin;
  // split partials (num_splits > 1): o_part [B, Hq, S, d_v] fp32, lse_part [B, Hq, S] (log2 units)
  float *o_part;
  float *lse_part;
  // paged cache (block_table != nullptr): key t of sequence b is row t & (2^page_shift - 1) of
  // page block_table[b * pages_per_seq + (t >> page_shift)]; k_sb / v_sb are the page strides.
  const int32_t *block_table;
  int page_shift;
  int pages_per_seq;
  // sliding window (> 0): sequence b sees keys max(0, kv_len - window) ..; split s of it covers
  // tiles first_tile + s * tiles_per_split .. (first_tile = that key / B_c). 0 = none.
  int window;
};

hipError_t launch_decode_gqa(const DecodeParams &p, int head_dim, hipStream_t stream);
hipError_t launch_decode_mla(const DecodeParams &p, hipStream_t stream);
// MLA with up to 128 query heads per unit (mla128.hip).
hipError_t launch_decode_mla128(const DecodeParams &p, hipStream_t stream);
hipError_t launch_split_combine(const DecodeParams &p, int head_dim_v, hipStream_t stream);

}  // namespace blasst

// Host path of a decode call, shared by blasst_attn_decode (caller's workspace) and
// blasst_attn_decode_noalloc (the library's scratch array); defined in api.cpp.
namespace blasst {
// Argument and plan checks of a decode call (host only; no HIP call).
blasst_status decode_check(const blasst_decode_args *a);
// Checks, plans and launches a decode call with the given split workspace.
blasst_status decode_with_workspace(const blasst_decode_args *a, void *workspace,
                                    size_t workspace_bytes, void *stream);
}  // namespace blasst

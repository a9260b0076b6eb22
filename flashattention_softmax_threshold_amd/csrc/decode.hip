// decode.hip -- BLASST skip-softmax decode for GQA / MQA on gfx950, and the split merge.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm" (per-tile test on
// tile_max - running_max < ln lambda over every query row of the tile). Decode follows the
// BLASST talk notes ("kernel design: decode"): decode is bound by reading the KV cache, so a
// skipped tile must not load its V tile at all; the K tiles of a batch are loaded back to back,
// the test is taken for all of them, and only the surviving V tiles are requested.
//
// Work unit (one workgroup, 4 waves): (split, KV head g, block of up to RB query heads that share
// g, sequence b); the rows of a tile are those query heads. A "round" is 4 consecutive key tiles,
// one per wave. Every K and V tile goes from HBM straight into the wave's own LDS tiles
// (global_load_lds_dwordx4), so no load is visible to the compiler and every wait is an explicit
// count of the wave's copies in flight:
//   1. each wave computes S^T = K Q^T for its tile with v_mfma_f32_16x16x32_bf16, K read from its
//      LDS tile; then it requests the K tile of the next round into the same LDS tile;
//   2. tile row maxima meet in LDS; every wave forms the same running (prefix) maxima over the 4
//      tiles in key order, the same per-tile votes and the round maximum M;
//   3. the wave accumulates O^T += V^T P^T for its kept tile of the PREVIOUS round (V^T read from
//      its LDS V tile with ds_read_b64_tr_b16, P kept in registers in the B operand layout of the
//      16x16x32 MFMA); O and l move to M; if this round's tile is kept it forms P = exp2(S - M)
//      in bf16 and only now requests its V tile. Skipped tiles load no V at all.
//   4. at the end the 4 waves' partial O and l are summed through LDS.
// A kept tile's V is thus consumed one round after it is requested, behind the next round's
// scores and vote, instead of being waited for in the round that asked for it; the terms enter O
// in the same order as when each round consumed its own V (bit-identical results).
// Using the round maximum M for P (instead of re-scaling tile by tile) is the same online
// softmax in exact arithmetic; the skip decisions use each tile's own prefix maximum.
#include "internal.h"
#include "lds_dma.h"

#include <math.h>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Waits until at most N of this wave's vector memory loads are outstanding (s_waitcnt with
// vmcnt = N; the export and LDS counters are left at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// LDS holds a K and a V tile per wave: 128 KiB per workgroup at d = 128 (one workgroup per CU,
// each wave with up to 32 KiB of copies in flight), 64 KiB at d = 64 (two per CU).
template <int D, int RB, bool PAGED>
__global__ __launch_bounds__(256, D == 64 ? 2 : 1) void decode_gqa_kernel(DecodeParams p) {
  constexpr int STEPS = D / 32;  // k-steps of one 16x16x32 MFMA chain
  constexpr int CPR = D / 8;     // 16-byte chunks per key row
  constexpr int ROWB = 2 * D;    // bytes of a key row
  constexpr int RPL = 1024 / ROWB;            // key rows one wave-wide 16-byte copy fills
  constexpr int NLD = kBlockC / RPL;          // copies per wave per K or V tile
  constexpr int RPB = 256 / ROWB;             // key rows per 256 bytes of LDS banks
  // Each wave's K and V tiles (64 keys x D, bf16) in LDS, 16-byte chunks XOR-swizzled by the
  // row; the V tiles' memory holds the waves' partial O for the final sum.
  __shared__ __attribute__((aligned(1024))) char sK[4][kBlockC * ROWB];
  __shared__ __attribute__((aligned(1024))) char sV[4][kBlockC * ROWB];
  static_assert(sizeof(float) * 4 * RB * D <= sizeof(sV), "partial O must fit in the V tiles");
  float(*sO)[RB][D] = reinterpret_cast<float(*)[RB][D]>(&sV[0][0]);
  __shared__ float sT[2][4][16];
  __shared__ float sL[4][16];
  __shared__ float sM[16];
  // Chunk c of key row r sits at chunk c ^ vswz(r): 8 consecutive rows reading the same
  // 32-byte column window (a transposing read) cover all 64 banks.
  auto vswz = [&](int r) { return 2 * ((r / RPB) % (CPR / 2)); };
  // K: chunk c of row r at c ^ (r % CPR): the 16 rows of one score k-step read 16 distinct
  // 16-byte bank slots.
  auto kswz = [&](int r) { return r & (CPR - 1); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15;     // S^T column = query row
  const int kgrp = lane >> 4;  // which 8 of the 32 k values / which 4 keys of a 16-key block
  const int split = blockIdx.x;
  const int g = blockIdx.y / p.n_rblocks;
  const int rb = blockIdx.y % p.n_rblocks;
  const int b = blockIdx.z;
  const int h0 = g * p.group + rb * p.block_r;
  const int nrows = min(p.block_r, p.group - rb * p.block_r);
  int seq_len = p.kv_len ? p.kv_len[b] : p.max_kv_len;
  seq_len = max(0, min(seq_len, p.max_kv_len));
  const int seq_tiles = (seq_len + kBlockC - 1) / kBlockC;
  // Sliding window: the query sees keys from seq_len - window on; the splits cut the tiles from
  // the one holding that key.
  const int first_key = p.window > 0 ? max(0, seq_len - p.window) : 0;
  const int t_base = first_key / kBlockC;
  const int t_begin = t_base + split * p.tiles_per_split;
  const int t_split_end = min(t_begin + p.tiles_per_split, p.n_tiles);
  const int t_end = min(t_split_end, seq_tiles);

  // Row of key `key` of this sequence and KV head: contiguous (base + key * row stride) or, for
  // a paged cache, row key % page_size of page block_table[b][key / page_size] (the batch stride
  // is then the page stride). Only keys below seq_len are ever addressed.
  const __bf16 *__restrict__ Kg =
      (const __bf16 *)p.k + (PAGED ? 0 : b * p.k_sb) + g * p.k_sh;
  const __bf16 *__restrict__ Vg =
      (const __bf16 *)p.v + (PAGED ? 0 : b * p.v_sb) + g * p.v_sh;
  // Paged: each lane holds the page of key `lane` of a tile, read two rounds before the tile's
  // copies are issued (the compiler waits for such a read, and with it for every copy issued
  // before it, before the page is first used); a row's page comes from the lane that holds it
  // with one cross-lane read.
  const int32_t *__restrict__ bt = PAGED ? p.block_table + (int64_t)b * p.pages_per_seq : nullptr;
  const int pmask = (1 << p.page_shift) - 1;
  auto page_of_lane_key = [&](int tile) -> int {  // page of key tile * 64 + lane (clamped)
    if constexpr (PAGED) {
      const int key = min(tile * kBlockC + lane, seq_len - 1);
      return bt[key >> p.page_shift];
    } else {
      return 0;
    }
  };
  auto row_off = [&](int key, int pages, int64_t sb, int64_t ss) -> int64_t {
    if constexpr (PAGED) {
      const int pg = __shfl(pages, key & (kBlockC - 1));
      return (int64_t)pg * sb + (int64_t)(key & pmask) * ss;
    } else {
      return (int64_t)key * ss;
    }
  };
  int pages_cur = 0, pages_next = 0, pages_nn = 0;  // paged: the tiles of rounds r, r + 1, r + 2
  const int64_t unit_tiles =
      (((int64_t)b * p.Hkv + g) * p.n_rblocks + rb) * (int64_t)p.n_tiles;

  // Q fragments: B operand (k = head dim, n = query row); rows past nrows are zero.
  bf16x8_t qf[STEPS];
  {
    const bool ok = n < nrows;
    const __bf16 *qrow = (const __bf16 *)p.q + b * p.q_sb + (int64_t)(h0 + (ok ? n : 0)) * p.q_sh;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
      qf[s] = ok ? *(const bf16x8_t *)(qrow + 32 * s + 8 * kgrp) : (bf16x8_t)(__bf16)0.f;
  }

  // K and V copies, straight from HBM into this wave's LDS tiles (global_load_lds_dwordx4): lane L
  // of copy kk fills row kk * RPL + L / CPR at physical chunk L % CPR with logical chunk
  // (L % CPR) ^ swizzle(row); keys past the sequence copy its last row (their scores are masked
  // and their P is 0).
  const uint32_t sk_base = lds_addr(&sK[wv][0]);
  const uint32_t sv_base = lds_addr(&sV[wv][0]);
  auto copy_tile = [&](const __bf16 *base, int64_t sb, int64_t ss, int t, int pages,
                       uint32_t lds, bool is_v) {
#pragma unroll
    for (int kk = 0; kk < NLD; ++kk) {
      const int r = kk * RPL + lane / CPR;
      const int key = min(t * kBlockC + r, seq_len - 1);
      const int64_t off = row_off(key, pages, sb, ss);
      const int sw = is_v ? vswz(r) : kswz(r);
      lds_dma16(base + off + 8 * ((lane % CPR) ^ sw), lds + kk * 1024);
    }
  };
  auto load_k = [&](int t, int pages) { copy_tile(Kg, p.k_sb, p.k_ss, t, pages, sk_base, false); };
  auto load_v = [&](int t, int pages) { copy_tile(Vg, p.v_sb, p.v_ss, t, pages, sv_base, true); };
  // K operand of S^T = K Q^T (16 keys x 32 head dims per MFMA): lane (n, kgrp) reads key
  // 16 kb + n, logical chunk 4 s + kgrp.
  auto rdk = [&](int kb, int s) {
    const int r = 16 * kb + n;
    return *(const bf16x8_t *)(&sK[wv][r * ROWB + 16 * ((4 * s + kgrp) ^ kswz(r))]);
  };

  // O^T = V^T P^T on the matrix cores: oacc[db] holds head dims 16 db + 4 kgrp .. + 3 of query
  // row n (16x16 output blocks).
  f32x4_t oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = (f32x4_t)0.f;
  // Transposing V reads: for k-step ks (keys 32 ks ..) and column block db, source lane L points at
  // key 32 ks + 4 (L / 16) + (L % 16) / 4 (+ 16 for the second read), head dims
  // 16 db + 4 (L % 4) .. + 3; lane L then receives head dim 16 db + L % 16 at the keys
  // 32 ks + 4 (L / 16) + 0..3 (and + 16), the key order of the P fragments.
  const int tr_row = 4 * (lane >> 4) + ((lane & 15) >> 2);
  const int tr_cb = lane & 3;
  bf16x8_t pb[2];  // P of this wave's last kept tile: B operands of its two 32-key k-steps
  auto pv = [&]() {
    const char *vt = &sV[wv][0];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const int r0 = 32 * ks + tr_row, r1 = r0 + 16;
        const int c = 2 * db + (tr_cb >> 1);
        const char *p0 = vt + r0 * ROWB + 16 * (c ^ vswz(r0)) + 8 * (tr_cb & 1);
        const char *p1 = vt + r1 * ROWB + 16 * (c ^ vswz(r1)) + 8 * (tr_cb & 1);
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
        const bf16x8_t va =
            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[ks], oacc[db], 0, 0, 0);
      }
    }
  };
  float l_part = 0.f;
  float m_run = -INFINITY;
  unsigned visited = 0, skipped = 0;
  const int n_rounds = t_end > t_begin ? (t_end - t_begin + 3) / 4 : 0;

  // Copy order of a wave: K of round 0; then per round r, K of round r + 1 (after the scores of
  // round r) and V of round r (after the vote, kept tiles only). So at the top of round r the
  // wave's outstanding copies are K_r and then (if its tile of round r - 1 was kept) V_{r-1}, and
  // at the P.V of round r - 1 they are V_{r-1} and then K_{r+1} (if any): the waits below count
  // copies accordingly (vmcnt counts this wave's loads, which complete in issue order).
  if (n_rounds > 0 && t_begin + wv < t_end) {
    pages_cur = page_of_lane_key(t_begin + wv);
    if (PAGED && t_begin + wv + 4 < t_end) pages_next = page_of_lane_key(t_begin + wv + 4);
    load_k(t_begin + wv, pages_cur);
  }
  bool pv_pending = false;  // the wave's tile of the previous round was kept: V in sV, P in pb

  for (int r = 0; r < n_rounds; ++r) {
    const int t = t_begin + 4 * r + wv;
    const bool have = t < t_end;
    if (pv_pending)
      wait_vmcnt<NLD>();  // K_r has landed; V_{r-1} may still be in flight
    else
      wait_vmcnt<0>();
    wave_lds_sync();
    if (PAGED && t + 8 < t_end) pages_nn = page_of_lane_key(t + 8);  // used two rounds on
    f32x4_t sacc[4];
    float mt = -INFINITY;
    const bool next_k = have && t + 4 < t_end;
    if (have) {
      if constexpr (PAGED) {
        // Paged: all 4 x STEPS K fragments are requested first and the MFMAs take them k-step by
        // k-step across the 4 key blocks (each block's sum keeps its order, so the result is the
        // same); faster by 2-3 % here, but slower by as much on a contiguous cache.
        bf16x8_t kf[4 * STEPS];
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) kf[4 * s + kb] = rdk(kb, s);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sacc[kb] = (f32x4_t)0.f;
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[4 * s + kb], qf[s], sacc[kb], 0, 0, 0);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          sacc[kb] = (f32x4_t)0.f;
#pragma unroll
          for (int s = 0; s < STEPS; ++s)
            sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rdk(kb, s), qf[s], sacc[kb], 0, 0, 0);
        }
      }
      if ((t + 1) * kBlockC > seq_len || t * kBlockC < first_key) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = t * kBlockC + 16 * kb + 4 * kgrp + i;
            if (key >= seq_len || key < first_key) sacc[kb][i] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mt = fmaxf(mt, sacc[kb][i]);
      // The next round's K goes into the same LDS tile: every read of this one has been
      // consumed by the MFMAs above.
      if (next_k) load_k(t + 4, pages_next);
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sacc[kb] = (f32x4_t)0.f;
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16));
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = (n < nrows) ? __fmul_rn(mt, p.scale_log2) : -INFINITY;
    if (lane < 16) sT[r & 1][wv][lane] = mt2;
    __syncthreads();

    // Prefix running maxima over the round's 4 tiles (key order) and the votes.
    float mp = m_run;
    bool keep_w[4];
    float dmy = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float tm = sT[r & 1][w][n];
      const float m2 = fmaxf(mp, tm);
      const float dl = (tm >= mp) ? 0.f : __fsub_rn(tm, mp);  // exactly 0 for a new row maximum
      const bool valid = (n < nrows) && tm > -INFINITY;
      keep_w[w] = __ballot(valid && !(dl < p.tau_log2)) != 0ull;
      if (w == wv) dmy = valid ? dl : -INFINITY;
      mp = m2;
    }
    const float M = mp;
    const bool my_keep = have && keep_w[wv];

    // P.V of the wave's kept tile of the previous round, into O still scaled to that round's max.
    if (pv_pending) {
      if (next_k)
        wait_vmcnt<NLD>();  // V_{r-1} has landed; K_{r+1} may still be in flight
      else
        wait_vmcnt<0>();
      wave_lds_sync();
      pv();
    }
    // A kept tile's V is requested now (the previous V tile's reads were consumed by pv() above)
    // and used next round.
    if (my_keep) load_v(t, pages_cur);
    // Move O and l to this round's max; a kept tile's P = exp2(S - M) in bf16 as the B operands
    // of its two 32-key k-steps (elements 0..3 are the keys of block 2 ks, 4..7 those of block
    // 2 ks + 1, this lane's 4 keys of each).
    const float M_use = (M == -INFINITY) ? 0.f : M;
    const float alpha = exp2_fast(m_run - M_use);  // for this lane's row n
    l_part *= alpha;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
    if (my_keep) {
      const bool row_live = n < nrows;
      const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
      float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = sacc[2 * ks + (e >> 2)][e & 3];
          pb[ks][e] = (__bf16)(row_live ? exp2_fast(fmaf(x, p.scale_log2, -M_use)) : 0.f);
        }
        const bf16x2_t x0 = {pb[ks][0], pb[ks][1]}, x1 = {pb[ks][2], pb[ks][3]};
        const bf16x2_t x2 = {pb[ks][4], pb[ks][5]}, x3 = {pb[ks][6], pb[ks][7]};
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(x0, one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(x1, one, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(x2, one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(x3, one, ps1, false);
      }
      l_part += ps0 + ps1;
    }
    pv_pending = my_keep;
    m_run = M;
    if constexpr (PAGED) {
      pages_cur = pages_next;
      pages_next = pages_nn;
    }

    if (have) {
      ++visited;
      skipped += my_keep ? 0u : 1u;
      if (p.tile_margin) {
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) dmy = fmaxf(dmy, __shfl_xor(dmy, off));
      }
      if (lane == 0) {
        if (p.tile_status) p.tile_status[unit_tiles + t] = my_keep ? 0 : 1;
        if (p.tile_margin) p.tile_margin[unit_tiles + t] = dmy * kLn2;
      }
    }
  }
  if (pv_pending) {  // the last kept tile's P.V
    wait_vmcnt<0>();
    wave_lds_sync();
    pv();
  }
  wait_vmcnt<0>();

  // ---- Sum the waves' partials; write O (unsplit) or the split's partial.
  __syncthreads();  // every wave's last V reads are done: the V tiles become sO
  if (n < RB) {
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) sO[wv][n][16 * db + 4 * kgrp + i] = oacc[db][i];
  }
  float lrow = l_part;
  lrow += __shfl_xor(lrow, 16);
  lrow += __shfl_xor(lrow, 32);
  if (lane < 16) sL[wv][lane] = lrow;
  if (wv == 0 && lane < 16) sM[lane] = m_run;  // every wave holds the same running maxima
  __syncthreads();

  for (int idx = tid; idx < nrows * D; idx += 256) {
    const int rr = idx / D, d = idx % D;
    const float L = sL[0][rr] + sL[1][rr] + sL[2][rr] + sL[3][rr];
    const float acc = sO[0][rr][d] + sO[1][rr][d] + sO[2][rr][d] + sO[3][rr][d];
    const float val = L > 0.f ? acc / L : 0.f;
    const float m_row = sM[rr];
    const int h = h0 + rr;
    if (p.num_splits == 1) {
      ((__bf16 *)p.o)[b * p.o_sb + (int64_t)h * p.o_sh + d] = (__bf16)val;
      if (d == 0 && p.lse)
        p.lse[(int64_t)b * p.Hq + h] = L > 0.f ? (m_row + __log2f(L)) * kLn2 : -INFINITY;
    } else {
      const int64_t row = ((int64_t)b * p.Hq + h) * p.num_splits + split;
      p.o_part[row * D + d] = val;
      if (d == 0) p.lse_part[row] = L > 0.f ? m_row + __log2f(L) : -INFINITY;
    }
  }
  if (lane == 0 && p.counters && visited) {
    atomicAdd(&p.counters[0], (unsigned long long)visited);
    atomicAdd(&p.counters[1], (unsigned long long)skipped);
  }
  if (tid == 0 && (p.tile_status || p.tile_margin)) {
    // Not visited: the rest of this split's range past the sequence; with a window, split 0
    // also marks the tiles before it and the last split those after every split's range.
    const int cover_end = min(t_base + p.num_splits * p.tiles_per_split, p.n_tiles);
    for (int t = 0; t < p.n_tiles; ++t) {
      const bool mine = (t >= max(t_begin, t_end) && t < t_split_end) ||
                        (split == 0 && t < t_base) ||
                        (split == p.num_splits - 1 && t >= cover_end);
      if (!mine) continue;
      if (p.tile_status) p.tile_status[unit_tiles + t] = 2;
      if (p.tile_margin) p.tile_margin[unit_tiles + t] = -INFINITY;
    }
  }
}

// Merge of split partials by log-sum-exp ("The Hitchhiker's Guide", LSE output L = m + log l:
// exp(L_s) is split s's softmax denominator). lse_part is in base-2 units.
__global__ __launch_bounds__(128) void split_combine_kernel(DecodeParams p, int dv) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int S = p.num_splits;
  const int64_t row0 = ((int64_t)b * p.Hq + h) * S;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, p.lse_part[row0 + s]);
  float wsum = 0.f;
  for (int s = 0; s < S; ++s) {
    const float x = p.lse_part[row0 + s];
    if (x > -INFINITY) wsum += exp2_fast(x - M);
  }
  // dv is 64, 128 or 512: each thread merges 4 consecutive columns with 16-byte reads.
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  for (int d = 4 * (int)threadIdx.x; d < dv; d += 4 * (int)blockDim.x) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const float x = p.lse_part[row0 + s];
      if (x > -INFINITY) {
        const float w = exp2_fast(x - M);
        const float4 v = *(const float4 *)(p.o_part + (row0 + s) * dv + d);
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
      }
    }
    const bool any = M > -INFINITY;
    const bf16x4_t ov = {(__bf16)(any ? acc.x / wsum : 0.f), (__bf16)(any ? acc.y / wsum : 0.f),
                         (__bf16)(any ? acc.z / wsum : 0.f), (__bf16)(any ? acc.w / wsum : 0.f)};
    *(bf16x4_t *)((__bf16 *)p.o + b * p.o_sb + (int64_t)h * p.o_sh + d) = ov;
  }
  if (threadIdx.x == 0 && p.lse)
    p.lse[(int64_t)b * p.Hq + h] = M > -INFINITY ? (M + __log2f(wsum)) * kLn2 : -INFINITY;
}

template <int D, bool PAGED>
hipError_t launch_gqa_dp(const DecodeParams &p, hipStream_t stream) {
  const dim3 grid(p.num_splits, p.Hkv * p.n_rblocks, p.B);
  if (p.block_r <= 4)
    hipLaunchKernelGGL((decode_gqa_kernel<D, 4, PAGED>), grid, dim3(256), 0, stream, p);
  else if (p.block_r <= 8)
    hipLaunchKernelGGL((decode_gqa_kernel<D, 8, PAGED>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_gqa_kernel<D, 16, PAGED>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_gqa_d(const DecodeParams &p, hipStream_t stream) {
  return p.block_table ? launch_gqa_dp<D, true>(p, stream) : launch_gqa_dp<D, false>(p, stream);
}

}  // namespace

hipError_t launch_decode_gqa(const DecodeParams &p, int head_dim, hipStream_t stream) {
  if (head_dim == 128) return launch_gqa_d<128>(p, stream);
  if (head_dim == 64) return launch_gqa_d<64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_split_combine(const DecodeParams &p, int head_dim_v, hipStream_t stream) {
  hipLaunchKernelGGL(split_combine_kernel, dim3(p.Hq, p.B), dim3(128), 0, stream, p, head_dim_v);
  return hipGetLastError();
}

}  // namespace blasst

// prefill_mfma.hip -- the bf16 BLASST prefill kernel for gfx950 with B_r = 128 query rows.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm": FlashAttention's streaming pass
// over key tiles in ascending order ("The Hitchhiker's Guide -- Phase 08", Section 1), where a
// tile's softmax and P.V are skipped when tile_max - running_max < ln(lambda) for every query row
// of the tile. As in the BLASST talk notes ("kernel design: prefill"), V is loaded whatever the
// test says (prefill is not bandwidth-bound and a predictable prefetch beats a conditional one);
// the exp / rescale / P.V MFMA work is what a skipped tile saves.
//
// Data path (one workgroup = 4 waves = one unit of 128 query rows; a wave owns 32 rows):
//   * K and V tiles (64 keys x D, bf16) go from HBM/L2 straight into LDS with
//     global_load_lds_dwordx4 (no registers, no LDS store instructions), two stages deep: the
//     next tile is in flight while the current one is used.
//   * LDS rows are stored unpadded; the 16-byte chunks of a row are XOR-swizzled so the MFMA
//     operand reads spread over all banks (K: chunk ^ (row % chunks_per_row); V: chunk ^
//     4 * (row % 4)). The swizzle is applied by choosing, per lane, which global chunk to load.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = the wave's Q rows kept in
//     registers): a lane holds 32 scores of one query row, so row max, running max and row sum
//     are per-lane values.
//   * O^T = V^T P^T: P comes straight from the S accumulators (bf16); the V^T operand is read
//     from the row-major V tile with ds_read_b64_tr_b16 (two per MFMA), whose 16-lane transpose
//     hands each lane the 8 keys of one column in the accumulator's key order.
//   * Skip vote: each row votes keep iff it is valid, sees a key of the tile and its margin is
//     not below tau; a wave ballots, the 4 waves meet through LDS and a barrier, and the branch
//     is uniform over the workgroup.
// Block order: units of one KV head are numbered (query block longest-first, then query head),
// and blocks are dealt to the 8 XCDs so each XCD works through contiguous runs of units: the
// query heads that share K/V read it through the same L2 at about the same time.
#include "internal.h"

#include <math.h>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBR = 128;  // query rows per workgroup
constexpr int kNW = 4;    // waves per workgroup
constexpr int kNT = 64 * kNW;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <int D>
struct Geo {
  static constexpr int ROW_BYTES = D * 2;                  // one key row of K or V
  static constexpr int CPR = D / 8;                        // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;   // rows one wave-wide 16-byte load fills
  static constexpr int TILE_BYTES = kBlockC * ROW_BYTES;
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / kNW;
  static constexpr int SWZ_V_MASK = CPR - 1;
};

__device__ __forceinline__ int swz_k(int row, int cpr) { return row & (cpr - 1); }
__device__ __forceinline__ int swz_v(int row, int cpr) { return (4 * (row & 3)) & (cpr - 1); }

template <int D>
__global__ __launch_bounds__(kNT, 2) void prefill_mfma_kernel(PrefillParams p) {
  using G = Geo<D>;
  constexpr int RB = G::ROW_BYTES, CPR = G::CPR;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][G::TILE_BYTES];  // [stage][K,V]
  __shared__ int sVote[kNW];
  __shared__ float sMargin[kNW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;

  // ---- Which unit: XCD-aware numbering (see the header comment).
  const int grp = p.Hq / p.Hkv;
  const int n_units = p.B * p.Hq * p.n_qblocks;
  int u = (int)blockIdx.x;
  if ((n_units & 7) == 0) u = (u & 7) * (n_units >> 3) + (u >> 3);
  const int per_kv = grp * p.n_qblocks;
  const int bg = u / per_kv;          // b * Hkv + g
  const int t = u - bg * per_kv;
  const int qb_r = t / grp;
  const int hl = t - qb_r * grp;
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int hq = g * grp + hl;
  const int qb = p.causal ? (p.n_qblocks - 1 - qb_r) : qb_r;

  const __bf16 *__restrict__ Qg = (const __bf16 *)p.q + b * p.q_sb + hq * p.q_sh;
  const __bf16 *__restrict__ Kg = (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh;
  const __bf16 *__restrict__ Vg = (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh;
  const int blk_row0 = qb * kBR;
  const int my_row = blk_row0 + wv * 32 + n;
  const bool row_ok = my_row < p.Lq;
  int n_tiles = p.n_kvtiles;
  if (p.causal) n_tiles = (min(blk_row0 + kBR, p.Lq) - 1) / kBlockC + 1;

  // ---- Q fragments: B operand of S^T = K Q^T (k = head dim, n = query row).
  bf16x8_t qf[D / 16];
  {
    const __bf16 *qrow = Qg + (int64_t)(row_ok ? my_row : 0) * p.q_ss;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = row_ok ? *(const bf16x8_t *)(qrow + 16 * s + 8 * hh) : (bf16x8_t)(__bf16)0.f;
  }

  // ---- Tile loads straight into LDS. Wave wv fills rows
  // [wv * LOADS_PER_WAVE * ROWS_PER_LOAD, ...) of each operand; lane L of a load fills row
  // r0 + L / CPR at chunk position L % CPR, fetching logical chunk (L % CPR) ^ swizzle(row).
  const int ld_row_in = lane / CPR;
  const int ld_pc = lane % CPR;
  auto issue_tile = [&](int j, int st) {
    const int k0 = j * kBlockC;
#pragma unroll
    for (int t2 = 0; t2 < G::LOADS_PER_WAVE; ++t2) {
      const int ii = wv * G::LOADS_PER_WAVE + t2;
      const int r = ii * G::ROWS_PER_LOAD + ld_row_in;
      const int key = min(k0 + r, p.Lkv - 1);  // rows past the end load a real row; masked later
      const __bf16 *kp = Kg + (int64_t)key * p.k_ss + 8 * (ld_pc ^ swz_k(r, CPR));
      const __bf16 *vp = Vg + (int64_t)key * p.v_ss + 8 * (ld_pc ^ swz_v(r, CPR));
      __builtin_amdgcn_global_load_lds((const void *)kp, (lds_void_t *)(&smem[st][0][ii * 1024]),
                                       16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void *)vp, (lds_void_t *)(&smem[st][1][ii * 1024]),
                                       16, 0, 0);
    }
  };

  // Per-lane LDS offsets of the MFMA operands.
  // K (A operand of S^T): row 32 kb + n, logical chunk 2 s + hh.
  const int k_rowoff = n * RB;
  const int k_swz = swz_k(n, CPR);  // (32 kb + n) % CPR == n % CPR
  // V^T via transpose reads: as a source lane, this lane points at row 16 s + 4 (lane / 32) +
  // (lane % 16) / 4 (+ 8 for the second read) and columns 32 db + 16 ((lane / 16) % 2) +
  // 4 (lane % 4) .. + 3.
  const int v_jj = (lane & 15) >> 2;
  const int v_rowoff = (4 * (lane >> 5) + v_jj) * RB;
  const int v_cb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int v_swz = (4 * v_jj) & (CPR - 1);
  const int v_byte = 8 * (lane & 1);

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16_t)0.f;
  float m_run = -INFINITY;
  float l_part = 0.f;
  unsigned visited = 0, skipped = 0;
  const int64_t unit_tiles =
      (((int64_t)b * p.Hq + hq) * p.n_qblocks + qb) * (int64_t)p.n_kvtiles;

  issue_tile(0, 0);

  for (int j = 0; j < n_tiles; ++j) {
    const int st = j & 1;
    const int k0 = j * kBlockC;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's part of tile j has landed in LDS
    __syncthreads();                // ... and every wave's; stage st ^ 1 is free again
    if (j + 1 < n_tiles) issue_tile(j + 1, st ^ 1);

    // ---- S^T = K Q^T (always: the test needs the scores).
    f32x16_t sacc[2];
    sacc[0] = (f32x16_t)0.f;
    sacc[1] = (f32x16_t)0.f;
    const char *kl = smem[st][0];
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t a = *(const bf16x8_t *)(kl + kb * 32 * RB + k_rowoff +
                                               16 * ((2 * s + hh) ^ k_swz));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
      }
    }

    // ---- Mask: keys past the end, and (causal) keys after the row's position.
    const bool need_mask = (k0 + kBlockC > p.Lkv) || (p.causal && k0 + kBlockC - 1 > blk_row0);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= p.Lkv || (p.causal && key > my_row)) sacc[kb][i] = -INFINITY;
        }
      }
    }

    // ---- Tile row max, margin, vote. The margin is exactly 0 for a tile holding a new row
    // maximum (mt2 rounded on its own, no fused multiply-add with the subtraction).
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    const float mt2 = __fmul_rn(mt, p.scale_log2);
    const float m_new = fmaxf(m_run, mt2);
    const float delta = (mt2 >= m_run) ? 0.f : __fsub_rn(mt2, m_run);
    const bool has_key = mt2 > -INFINITY;
    const bool keep_row = row_ok && has_key && !(delta < p.tau_log2);
    const unsigned long long ballot = __ballot(keep_row);
    if (p.tile_margin) {
      float dm = (row_ok && has_key) ? delta : -INFINITY;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dm = fmaxf(dm, __shfl_xor(dm, o));
      if (lane == 0) sMargin[wv] = dm;
    }
    if (lane == 0) sVote[wv] = ballot != 0ull;
    __syncthreads();
    const int keep = sVote[0] | sVote[1] | sVote[2] | sVote[3];
    if (tid == 0) {
      ++visited;
      skipped += keep ? 0u : 1u;
      if (p.tile_status) p.tile_status[unit_tiles + j] = keep ? 0 : 1;
      if (p.tile_margin) {
        const float dm = fmaxf(fmaxf(sMargin[0], sMargin[1]), fmaxf(sMargin[2], sMargin[3]));
        p.tile_margin[unit_tiles + j] = dm * kLn2;
      }
    }

    if (keep) {
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float psum = 0.f;
      bf16x8_t pf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float pv = exp2_fast(fmaf(sacc[kb][i], p.scale_log2, -m_use));
          psum += pv;
          pf[kb * 2 + (i >> 3)][i & 7] = (__bf16)pv;
        }
      }
      l_part = fmaf(l_part, alpha, psum);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
      const char *vl = smem[st][1];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int coff = 16 * ((4 * db + v_cb) ^ v_swz) + v_byte;
          const char *p0 = vl + 16 * s * RB + v_rowoff + coff;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p0 + 8 * RB));
          const bf16x8_t a = __builtin_bit_cast(
              bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- Epilogue: O = acc / l, LSE = m + log l (natural log on output).
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    __bf16 *orow = (__bf16 *)p.o + b * p.o_sb + (int64_t)my_row * p.o_ss + hq * p.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = db * 32 + 8 * ig + 4 * hh;
        bf16x4_t ov = {(__bf16)(oacc[db][4 * ig + 0] * inv), (__bf16)(oacc[db][4 * ig + 1] * inv),
                       (__bf16)(oacc[db][4 * ig + 2] * inv), (__bf16)(oacc[db][4 * ig + 3] * inv)};
        *(bf16x4_t *)(orow + d0) = ov;
      }
    }
    if (p.lse && hh == 0) {
      p.lse[((int64_t)b * p.Hq + hq) * p.Lq + my_row] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  if (tid == 0) {
    if (p.counters) {
      atomicAdd(&p.counters[0], (unsigned long long)visited);
      atomicAdd(&p.counters[1], (unsigned long long)skipped);
    }
    if (p.tile_status || p.tile_margin) {
      for (int j = n_tiles; j < p.n_kvtiles; ++j) {
        if (p.tile_status) p.tile_status[unit_tiles + j] = 2;
        if (p.tile_margin) p.tile_margin[unit_tiles + j] = -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams &p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hq * p.n_qblocks));
  if (head_dim == 128)
    hipLaunchKernelGGL((prefill_mfma_kernel<128>), grid, dim3(kNT), 0, stream, p);
  else if (head_dim == 64)
    hipLaunchKernelGGL((prefill_mfma_kernel<64>), grid, dim3(kNT), 0, stream, p);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace blasst

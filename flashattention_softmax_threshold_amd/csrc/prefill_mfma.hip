// prefill_mfma.hip -- the bf16 BLASST prefill kernel for gfx950 with B_r = 128 query rows.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm": FlashAttention's streaming pass
// over key tiles in ascending order ("The Hitchhiker's Guide -- Phase 08", Section 1), where a
// tile's softmax and P.V are skipped when tile_max - running_max < ln(lambda) for every query row
// of the tile. As in the BLASST talk notes ("kernel design: prefill"), V is loaded whatever the
// test says (prefill is not bandwidth-bound and a predictable prefetch beats a conditional one);
// the exp / rescale / P.V MFMA work is what a skipped tile saves.
//
// Data path (one unit = 4 waves = 128 query rows, a wave owns 32 rows; a workgroup runs one unit,
// or two that share every K and V tile):
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
//     not below tau; a wave ballots, the unit's 4 waves meet through LDS and a barrier, and the
//     branch is uniform over the unit.
// Block order: units of one KV head are numbered (query block longest-first, then query head),
// and blocks are dealt to the 8 XCDs so each XCD works through contiguous runs of units: the
// query heads that share K/V read it through the same L2 at about the same time.
#include "internal.h"
#include "lds_dma.h"

#include <math.h>

#include <type_traits>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBR = 128;  // query rows per workgroup
constexpr int kNW = 4;    // waves per workgroup
constexpr int kNT = 64 * kNW;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Lanes l and l ^ 32 hold the two halves of one query row; v_permlane32_swap exchanges the wave's
// halves in one VALU op (no LDS round trip).
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max of the 32 scores a lane holds: a tree of three-input maxima (v_max3_f32), 16 VALU ops.
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
__device__ __forceinline__ float max32(const f32x16_t &a, const f32x16_t &b) {
  float m[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) m[i] = max3f(a[3 * i], a[3 * i + 1], a[3 * i + 2]);
#pragma unroll
  for (int i = 0; i < 5; ++i) m[5 + i] = max3f(b[3 * i], b[3 * i + 1], b[3 * i + 2]);
  m[10] = fmaxf(a[15], b[15]);
  const float x = max3f(m[0], m[1], m[2]), y = max3f(m[3], m[4], m[5]);
  const float z = max3f(m[6], m[7], m[8]);
  return max3f(max3f(x, y, z), m[9], m[10]);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// O and l are rescaled only when some row's max has grown by more than this (base-2 units)
// since the last rescale: P = 2^(s - m_ref) then stays below 2^8, and the algebra is exact.
constexpr float kRescaleSlack = 8.f;


template <int D, int NH>
struct Geo {
  static constexpr int ROW_BYTES = D * 2;                  // one key row of K or V
  static constexpr int CPR = D / 8;                        // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;   // rows one wave-wide 16-byte load fills
  static constexpr int TILE_BYTES = kBlockC * ROW_BYTES;
  static constexpr int LOADS_PER_WAVE = TILE_BYTES / 1024 / (kNW * NH);
  static constexpr int SWZ_V_MASK = CPR - 1;
};

__device__ __forceinline__ int swz_k(int row, int cpr) { return row & (cpr - 1); }
__device__ __forceinline__ int swz_v(int row, int cpr) { return (4 * (row & 3)) & (cpr - 1); }

// NH units per workgroup (4 waves, i.e. one 128-row unit, each) that read the same K and V
// tiles: NH query heads of one KV group at one query block, or, with QP (non-causal calls only),
// one query head at two neighbouring query blocks. The K and V tiles in LDS serve all NH units,
// so each wave issues 1 / NH of the loads. WIN: the call has a sliding window (a separate
// instance, so calls without one pay nothing for it).
template <int D, int NH, bool WIN, bool QP>
__global__ __launch_bounds__(kNT * NH, 2 / NH) void prefill_mfma_kernel(PrefillParams p) {
  using G = Geo<D, NH>;
  constexpr int RB = G::ROW_BYTES, CPR = G::CPR;
  __shared__ __attribute__((aligned(1024))) char smem[2][2][G::TILE_BYTES];  // [stage][K,V]
  __shared__ __attribute__((aligned(16))) int sVote[2][kNW * NH];  // [tile parity][wave]
  __shared__ float sMargin[2][kNW * NH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in a scalar
  const int hs = wv / kNW;  // which of the workgroup's heads
  const int wq = wv % kNW;  // wave within the head's unit
  const int n = lane & 31;
  const int hh = lane >> 5;

  // ---- Which unit: XCD-aware numbering (see the header comment).
  const int grp = p.Hq / p.Hkv;
  const int gw = QP ? grp : grp / NH;  // workgroups per (KV head, query block or block pair)
  const int n_qw = QP ? (p.n_qblocks + 1) / 2 : p.n_qblocks;  // query blocks (pairs) per head
  const int n_units = p.B * p.Hkv * gw * n_qw;
  int u = (int)blockIdx.x;
  if ((n_units & 7) == 0) u = (u & 7) * (n_units >> 3) + (u >> 3);
  const int per_kv = gw * n_qw;
  const int bg = u / per_kv;          // b * Hkv + g
  const int t = u - bg * per_kv;
  const int qb_r = t / gw;
  const int hl = t - qb_r * gw;
  const int b = bg / p.Hkv;
  const int g = bg - b * p.Hkv;
  const int hq = QP ? g * grp + hl : g * grp + hl * NH + hs;
  const int qb = QP ? 2 * qb_r + hs : (p.causal ? (p.n_qblocks - 1 - qb_r) : qb_r);
  // QP with an odd number of query blocks: the last pair's second unit does not exist (its rows
  // are all past Lq); its waves take part in the loads and barriers but record nothing.
  const bool unit_ok = qb < p.n_qblocks;

  const __bf16 *__restrict__ Qg = (const __bf16 *)p.q + b * p.q_sb + hq * p.q_sh;
  const __bf16 *__restrict__ Kg = (const __bf16 *)p.k + b * p.k_sb + g * p.k_sh;
  const __bf16 *__restrict__ Vg = (const __bf16 *)p.v + b * p.v_sb + g * p.v_sh;
  const int blk_row0 = qb * kBR;
  const int my_row = blk_row0 + wq * 32 + n;
  const bool row_ok = my_row < p.Lq;
  int n_tiles = p.n_kvtiles;
  if (p.causal) n_tiles = (min(blk_row0 + kBR, p.Lq) - 1) / kBlockC + 1;
  // Sliding window: the block's first row sees keys from blk_row0 - window + 1 on, so earlier
  // tiles are not visited.
  const int j0 = WIN ? max(0, blk_row0 - p.window + 1) / kBlockC : 0;

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
  // A lane's byte offset inside a tile is fixed, so it is computed once; per tile only the
  // scalar base moves (the host guarantees 64 rows of either stride fit in 32 bits), and the copy
  // takes it as a scalar base plus the lane's 32-bit offset (about 1 % faster than a 64-bit
  // address per lane).
  const int ld_row_in = lane / CPR;
  const int ld_pc = lane % CPR;
  uint32_t k_off[G::LOADS_PER_WAVE], v_off[G::LOADS_PER_WAVE];
#pragma unroll
  for (int t2 = 0; t2 < G::LOADS_PER_WAVE; ++t2) {
    const int r = (wv * G::LOADS_PER_WAVE + t2) * G::ROWS_PER_LOAD + ld_row_in;
    k_off[t2] = (uint32_t)(r * p.k_ss + 8 * (ld_pc ^ swz_k(r, CPR))) * 2u;
    v_off[t2] = (uint32_t)(r * p.v_ss + 8 * (ld_pc ^ swz_v(r, CPR))) * 2u;
  }
  // op 0 = K, 1 = V. Rows past the end of a partial last tile load a real row (masked later).
  auto issue = [&](int j, int st, int op) {
    const int k0 = j * kBlockC;
    const __bf16 *base = op ? Vg : Kg;
    const int64_t ss = op ? p.v_ss : p.k_ss;
    if (k0 + kBlockC <= p.Lkv) {
      const char *tb = (const char *)(base + (int64_t)k0 * ss);
#pragma unroll
      for (int t2 = 0; t2 < G::LOADS_PER_WAVE; ++t2) {
        const int ii = wv * G::LOADS_PER_WAVE + t2;
        lds_dma16_s(tb, op ? v_off[t2] : k_off[t2], lds_addr(&smem[st][op][ii * 1024]));
      }
    } else {
#pragma unroll
      for (int t2 = 0; t2 < G::LOADS_PER_WAVE; ++t2) {
        const int ii = wv * G::LOADS_PER_WAVE + t2;
        const int r = ii * G::ROWS_PER_LOAD + ld_row_in;
        const int key = min(k0 + r, p.Lkv - 1);
        const int sw = op ? swz_v(r, CPR) : swz_k(r, CPR);
        const __bf16 *gp = base + (int64_t)key * ss + 8 * (ld_pc ^ sw);
        lds_dma16(gp, lds_addr(&smem[st][op][ii * 1024]));
      }
    }
  };
  auto issue_k = [&](int j, int st) { issue(j, st, 0); };
  auto issue_v = [&](int j, int st) { issue(j, st, 1); };
  // Steps whose copies are all full tiles take them from running tile pointers (one 64-bit
  // scalar add per tile instead of a multiply and a bounds test per copy).
  const int n_full = p.Lkv / kBlockC;  // tiles with no row past the end
  const char *kt_run = (const char *)(Kg + (int64_t)(j0 + 2) * kBlockC * p.k_ss);
  const char *vt_run = (const char *)(Vg + (int64_t)(j0 + 1) * kBlockC * p.v_ss);
  const int64_t k_tile_bytes = (int64_t)kBlockC * p.k_ss * 2;
  const int64_t v_tile_bytes = (int64_t)kBlockC * p.v_ss * 2;
  auto issue_full = [&](const char *tb, int st, int op) {
#pragma unroll
    for (int t2 = 0; t2 < G::LOADS_PER_WAVE; ++t2) {
      const int ii = wv * G::LOADS_PER_WAVE + t2;
      lds_dma16_s(tb, op ? v_off[t2] : k_off[t2], lds_addr(&smem[st][op][ii * 1024]));
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
  float m_run = -INFINITY;  // running row max through the newest scored tile (base-2 units)
  float m_ref = -INFINITY;  // the max that O and l are currently scaled to
  float l_part = 0.f;       // this lane's share of the running row sum
  unsigned visited = 0, skipped = 0;
  const int64_t unit_tiles =
      (((int64_t)b * p.Hq + hq) * p.n_qblocks + qb) * (int64_t)p.n_kvtiles;

  // S^T = K Q^T for the tile in K stage st (always computed: the test needs the scores). The K
  // fragments are read from LDS KPF k-steps ahead of the MFMAs that use them, so LDS latency
  // hides behind matrix work; the scheduling hints keep that order. With vj >= 0 the copies of
  // V_vj and K_{vj+1} are issued between the MFMAs (after the second and the fourth k-step): a
  // wave held up issuing them still has MFMAs in flight.
  auto compute_s = [&](auto full_c, int st, f32x16_t *sacc, int vj = -1,
                       const int4 *votes = nullptr, int *vote_or = nullptr) {
    constexpr bool FULL = decltype(full_c)::value;
    constexpr int NS = D / 16;  // k-steps
    // The V copy goes out after k-step 1 and the K copy after k-step 3: both need four k-steps.
    static_assert(NS >= 4, "the in-loop copies need at least four k-steps (D >= 64)");
    constexpr int KPF = NS < 2 ? NS : 2;
    sacc[0] = (f32x16_t)0.f;
    sacc[1] = (f32x16_t)0.f;
    const char *kl = smem[st][0] + k_rowoff;
    bf16x8_t fr[NS][2];
    auto rd = [&](int s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        fr[s][kb] = *(const bf16x8_t *)(kl + kb * 32 * RB + 16 * ((2 * s + hh) ^ k_swz));
    };
#pragma unroll
    for (int s = 0; s < KPF; ++s) rd(s);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s + KPF < NS) rd(s + KPF);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s][kb], qf[s], sacc[kb], 0, 0, 0);
      // The unit's four vote words, read at the top of the step, folded into one wave-uniform
      // word behind the first k-step (so the vote read's wait does not hold up the first K
      // fragment reads, and only one scalar register carries it through the scores).
      if (s == 1 && votes)
        *vote_or = __builtin_amdgcn_readfirstlane(votes->x | votes->y | votes->z | votes->w);
      if constexpr (FULL) {
        if (s == 1) issue_full(vt_run, vj & 1, 1);
        if (s == 3) issue_full(kt_run, (vj + 1) & 1, 0);
      } else {
        if (s == 1 && vj >= 0) issue_v(vj, vj & 1);
        if (s == 3 && vj >= 0 && vj + 1 < n_tiles) issue_k(vj + 1, (vj + 1) & 1);
      }
    }
    // Scheduling: KPF steps of reads first, then (2 MFMAs, 2 reads) pairs, then the tail MFMAs.
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * KPF, 0);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      if (s + KPF < NS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Keys past the end, (causal) keys after the row's position and (window) keys before the
  // row's window score -inf.
  auto mask_tile = [&](int j, f32x16_t *sacc) {
    const int k0 = j * kBlockC;
    if ((k0 + kBlockC > p.Lkv) || (p.causal && k0 + kBlockC - 1 > blk_row0) ||
        (WIN && k0 <= blk_row0 + kBR - 1 - p.window)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= p.Lkv || (p.causal && key > my_row) ||
              (WIN && key <= my_row - p.window))
            sacc[kb][i] = -INFINITY;
        }
      }
    }
  };

  // Tile row max, margin and this wave's vote for tile j (published at the next barrier). The
  // running max does not depend on any skip decision, so it advances here. The margin is exactly
  // 0 for a tile holding a new row maximum (mt2 rounded on its own, no fused multiply-add).
  // Branch-free so it can share a basic block with the previous tile's softmax; every lane
  // writes the same wave vote. Returns the row's margin (-inf for a row that does not vote).
  auto vote_tile = [&](int j, const f32x16_t *sacc) {
    const float mt = max_halves(max32(sacc[0], sacc[1]));
    const float mt2 = __fmul_rn(mt, p.scale_log2);
    const float delta = (mt2 >= m_run) ? 0.f : __fsub_rn(mt2, m_run);
    m_run = fmaxf(m_run, mt2);
    const bool has_key = mt2 > -INFINITY;
    const bool keep_row = row_ok && has_key && !(delta < p.tau_log2);
    sVote[j & 1][wv] = __ballot(keep_row) != 0ull;
    return (row_ok && has_key) ? delta : -INFINITY;
  };
  // Optional observation: the wave's largest row margin for tile j.
  auto publish_margin = [&](int j, float dm) {
    if (p.tile_margin) {
      asm volatile("" : "+v"(dm));  // keeps the reduction inside the branch (no speculation)
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dm = fmaxf(dm, __shfl_xor(dm, o));
      sMargin[j & 1][wv] = dm;
    }
  };

  // The four votes of this head's unit (one 16-byte LDS read) and the unit's decision; the first
  // lane of the unit's first wave keeps its counts and observation outputs.
  const bool bookkeeper = wq == 0 && lane == 0 && unit_ok;
  auto read_votes = [&](int j) { return *(const int4 *)&sVote[j & 1][kNW * hs]; };
  auto decision = [&](int j, int keep) {
    if (bookkeeper) {
      ++visited;
      skipped += keep ? 0u : 1u;
      if (p.tile_status) p.tile_status[unit_tiles + j] = keep ? 0 : 1;
      if (p.tile_margin) {
        const float *sm = &sMargin[j & 1][kNW * hs];
        p.tile_margin[unit_tiles + j] = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3])) * kLn2;
      }
    }
    return keep;
  };

  // Online-softmax update for a kept tile whose running max (through the tile) is m_tile. O and
  // l stay scaled to m_ref until some row of the wave exceeds it by more than kRescaleSlack;
  // then every row of the wave moves to its own m_tile.
  auto rescale_to = [&](float m_tile) {
    if (__ballot(m_tile > m_ref + kRescaleSlack) != 0ull) {
      const float alpha = exp2_fast(m_ref - ((m_tile == -INFINITY) ? 0.f : m_tile));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_ref = m_tile;
    }
  };

  // O += P V for a kept tile: P = exp2(S - m_ref) in bf16 is the B operand of k-step s (keys
  // 16 s .. 16 s + 15: scores sacc[s / 2][8 (s % 2) ..]); the V^T A operands come from the
  // row-major V tile in stage st through ds_read_b64_tr_b16. Software-pipelined over the four
  // k-steps: the V reads of step s + 1 are in flight and the exponentials of step s + 1 are
  // computed while the MFMAs of step s run.
  auto exp_pv = [&](const f32x16_t *sacc, int st) {
    constexpr int NDB = D / 32;        // output column blocks
    constexpr int NM = 4 * NDB;        // MFMAs: (k-step s, column block db) = (m / NDB, m % NDB)
    constexpr int RA = 2;              // V operands read this many MFMAs ahead
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    const char *vl = smem[st][1];
    auto rdv = [&](int m) {
      const int s = m / NDB, db = m % NDB;
      const int coff = 16 * ((4 * db + v_cb) ^ v_swz) + v_byte;
      const char *p0 = vl + 16 * s * RB + v_rowoff + coff;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)(p0 + 8 * RB));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto mkp = [&](int s) {
      bf16x8_t pk;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        pk[i] = (__bf16)exp2_fast(fmaf(sacc[s >> 1][8 * (s & 1) + i], p.scale_log2, -m_use));
      return pk;
    };
    const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
    float ps0 = 0.f, ps1 = 0.f;
    bf16x8_t va[RA + 1];
    bf16x8_t pc = mkp(0), pn = pc;
#pragma unroll
    for (int m = 0; m < RA; ++m) va[m] = rdv(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int s = m / NDB, db = m % NDB;
      if (m + RA < NM) va[(m + RA) % (RA + 1)] = rdv(m + RA);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m % (RA + 1)], pc, oacc[db], 0, 0, 0);
      if (db == 0 && s < 3) pn = mkp(s + 1);
      if (db == NDB - 1) {
        const bf16x2_t x0 = {pc[0], pc[1]}, x1 = {pc[2], pc[3]};
        const bf16x2_t x2 = {pc[4], pc[5]}, x3 = {pc[6], pc[7]};
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(x0, one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(x1, one, ps1, false);
        ps0 = __builtin_amdgcn_fdot2_f32_bf16(x2, one, ps0, false);
        ps1 = __builtin_amdgcn_fdot2_f32_bf16(x3, one, ps1, false);
        pc = pn;
      }
    }
    l_part += ps0 + ps1;
    // Order: step-0 exponentials and the first V reads; then per MFMA the read RA ahead, the
    // MFMA, and a slice of the next step's VALU work.
    __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RA, 0);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + RA < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    }
  };

  // Software pipeline, one barrier per tile. Step j: the barrier publishes K_j, V_{j-1} and the
  // votes for tile j-1; the wave then scores tile j on the matrix cores while (if tile j-1 is
  // kept) it exponentiates tile j-1 and accumulates P_{j-1} V_{j-1}; finally it votes on tile j.
  // K_{j+1} and V_j are loaded meanwhile (two LDS stages each). The scores alternate between two
  // register sets, so no step copies them.
  auto step = [&](auto full_c, int j, f32x16_t *cur, const f32x16_t *prev) {
    constexpr bool FULL = decltype(full_c)::value;
    __builtin_amdgcn_s_waitcnt(0);  // this wave's K_j and V_{j-1} have landed
    __syncthreads();                // ... and every wave's; votes for tile j-1 are visible
    const int4 vt = read_votes(j - 1);
    // Copies of K_{j+1} and V_j: with two units per workgroup inside the S MFMAs (0.5 % faster
    // on causal GQA, 1.5 % on non-causal MHA with query-block pairs); with one unit up front
    // (inside, that kernel spills).
    if constexpr (NH == 1) {
      if (j + 1 < n_tiles) issue_k(j + 1, (j + 1) & 1);
      issue_v(j, j & 1);
    }
    const float m_prev = m_run;
    int vote_or = 0;
    compute_s(full_c, j & 1, cur, NH == 2 ? j : -1, &vt, &vote_or);
    if constexpr (FULL) {
      kt_run += k_tile_bytes;
      vt_run += v_tile_bytes;
    }
    // The decision on tile j - 1 is taken only now: the vote words are folded into one word
    // inside the scores, so the first K reads do not wait behind the vote read (one LDS round
    // trip at the top of the step instead of two) and the four words are not held through the
    // scores (which would push the two-unit kernel past 256 registers).
    const int keep_prev = decision(j - 1, vote_or);
    mask_tile(j, cur);
    if (keep_prev) {
      rescale_to(m_prev);
      // Two heads per workgroup: a wave in its exponential / P.V phase issues ahead of the other
      // head's wave on the same SIMD that is still scoring (about 1 % faster). With one head
      // per workgroup the two waves of a SIMD belong to different workgroups, and the same
      // priority costs 5 % at lambda = 0 (Video-DiT), so it is not raised there.
      if constexpr (NH == 2) __builtin_amdgcn_s_setprio(1);
      exp_pv(prev, (j - 1) & 1);
      if constexpr (NH == 2) __builtin_amdgcn_s_setprio(0);
    }
    publish_margin(j, vote_tile(j, cur));
  };
  auto finish = [&](const f32x16_t *last) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int4 vl = read_votes(n_tiles - 1);
    if (decision(n_tiles - 1, vl.x | vl.y | vl.z | vl.w)) {
      rescale_to(m_run);
      exp_pv(last, (n_tiles - 1) & 1);
    }
  };
  f32x16_t sa[2], sb[2];
  issue_k(j0, j0 & 1);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (n_tiles > j0 + 1) issue_k(j0 + 1, (j0 + 1) & 1);
  issue_v(j0, j0 & 1);
  compute_s(std::false_type{}, j0 & 1, sa);
  mask_tile(j0, sa);
  publish_margin(j0, vote_tile(j0, sa));
  int j = j0 + 1;
  // Two units per workgroup: pairs of steps whose copies (V_j, K_{j+1}, V_{j+1}, K_{j+2}) are
  // all full tiles first, then the rest. (The one-unit kernel keeps the general copies: the
  // extra loop copy there adds 4 bytes of spill.)
  if constexpr (NH == 2) {
    for (; j + 2 < n_tiles && j + 3 <= n_full; j += 2) {
      step(std::true_type{}, j, sb, sa);
      step(std::true_type{}, j + 1, sa, sb);
    }
  }
  for (; j + 1 < n_tiles; j += 2) {
    step(std::false_type{}, j, sb, sa);
    step(std::false_type{}, j + 1, sa, sb);
  }
  if (j < n_tiles) {
    step(std::false_type{}, j, sb, sa);
    finish(sb);
  } else {
    finish(sa);
  }

  // ---- Epilogue: O = acc / l, LSE = m + log l (natural log on output).
  const float l_tot = sum_halves(l_part);
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
          l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
  }
  if (bookkeeper) {
    if (p.counters) {
      atomicAdd(&p.counters[0], (unsigned long long)visited);
      atomicAdd(&p.counters[1], (unsigned long long)skipped);
    }
    if (p.tile_status || p.tile_margin) {
      for (int jt = 0; jt < p.n_kvtiles; ++jt) {
        if (jt >= j0 && jt < n_tiles) continue;
        if (p.tile_status) p.tile_status[unit_tiles + jt] = 2;
        if (p.tile_margin) p.tile_margin[unit_tiles + jt] = -INFINITY;
      }
    }
  }
}

}  // namespace

template <int D, int NH>
void launch_nh(const PrefillParams &p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hq / NH * p.n_qblocks));
  if (p.window > 0)
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NH, true, false>), grid, dim3(kNT * NH), 0, stream,
                       p);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<D, NH, false, false>), grid, dim3(kNT * NH), 0, stream,
                       p);
}

// Non-causal calls whose query heads do not pair up: two neighbouring query blocks of one head
// per workgroup.
template <int D>
void launch_qp(const PrefillParams &p, hipStream_t stream) {
  const dim3 grid((unsigned)(p.B * p.Hq * ((p.n_qblocks + 1) / 2)));
  hipLaunchKernelGGL((prefill_mfma_kernel<D, 2, false, true>), grid, dim3(kNT * 2), 0, stream, p);
}

// Two heads per workgroup when the query heads of a KV head pair up (even group), else one.
hipError_t launch_prefill_mfma(const PrefillParams &p, int head_dim, hipStream_t stream) {
  const bool pair = (p.Hq / p.Hkv) % 2 == 0;
  const bool qpair = !pair && !p.causal && p.window == 0 && p.n_qblocks > 1;
  if (head_dim == 128)
    pair ? launch_nh<128, 2>(p, stream)
         : (qpair ? launch_qp<128>(p, stream) : launch_nh<128, 1>(p, stream));
  else if (head_dim == 64)
    pair ? launch_nh<64, 2>(p, stream)
         : (qpair ? launch_qp<64>(p, stream) : launch_nh<64, 1>(p, stream));
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace blasst

// mla.hip -- MLA-shaped BLASST decode on gfx950: many query heads share one latent KV head,
// d_qk = 576, and V is the first 512 columns of K.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm": per key tile, skip the softmax
// and P.V when tile_max - running_max < ln(lambda) for every query row of the tile. The BLASST
// talk notes ("kernel design") observe that MLA decode can be compute-bound, so skipping the P.V
// work pays there even though V costs no extra traffic: the V tile is the K tile already on chip.
//
// Work unit (one workgroup of 4 waves): (sequence b, block of B_r = 64 heads, split of the key
// range). For the scores, wave w = (row group rg = w % 2, key half kh = w / 2) takes query heads
// 32 rg .. + 31 of the block against keys 32 kh .. + 31 of each tile; for P.V, wave w owns output
// columns 128 w .. + 127 of all 64 heads, so each V^T fragment it reads from LDS feeds two MFMAs
// (one per row group) and the four waves together read the V part of a tile once per row group
// pair instead of twice. Per key tile of 64 keys:
//   * the K tile (64 x 576 bf16, 72 KB) goes from HBM straight into LDS (global_load_lds_dwordx4,
//     two stages); the next tile's loads are issued between the MFMAs of this tile's scores;
//   * S^T (32 keys x 32 heads) = K Q^T with v_mfma_f32_32x32x16_bf16 over 36 k-steps: A = K rows
//     of the wave's key half from LDS, B = the wave's 32 query rows kept in registers (144 AGPRs);
//   * the waves publish their partial row maxima through LDS; after one barrier every wave forms
//     the tile maxima and running maxima of all 64 rows of the unit and takes the test itself,
//     so all four reach the same decision without exchanging votes;
//   * P = exp2(S - m_ref) of the wave's rows and key half goes to LDS before that barrier, formed
//     with the current reference max; for a kept tile each wave reads P of all 64 heads and keys
//     and accumulates O^T (128 x 64) += V^T P^T, V^T read from the same LDS tile with
//     ds_read_b64_tr_b16. (A kept tile that moves the reference max forms P again.)
// LDS layout: the latent parts of a tile's rows (64 x 1024 bytes) and their rotary parts
// (64 x 128 bytes) are stored apart, 16-byte chunks XOR-swizzled by the row so that the K and
// V^T reads are conflict-free. A wave-wide copy then moves either one latent row (1 KB of
// contiguous K: a wave-uniform row address plus the lane's swizzled chunk offset) or the rotary
// parts of 8 rows.
// Splits write normalised partial O and base-2 LSE to the workspace; the split merge combines.
#include "internal.h"
#include "lds_dma.h"

#include <math.h>

#include <type_traits>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;                 // 1152 bytes of a K row in HBM
constexpr int kLatBytes = kDv * 2;                  // 1024: the latent (V) part of a row
constexpr int kRopeBytes = kRowBytes - kLatBytes;   // 128: the rotary part
constexpr int kRopeOff = kBlockC * kLatBytes;       // 65536: rotary region of a stage
constexpr int kTileBytes = kBlockC * kRowBytes;     // 73728
constexpr int kLoadsPerTile = kTileBytes / 1024;    // 72 wave-wide 16-byte loads
constexpr int kRowLoads = kBlockC;                  // 64 of them copy one latent row each
constexpr int kSteps = kDqk / 16;                   // 36 k-steps of S
constexpr int kLatSteps = kDv / 16;                 // 32 of them over the latent part
constexpr int kDvBlocks = kDv / 32 / 4;             // 4 output column blocks per wave

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
// O and l are rescaled only when some row's max has grown by more than this (base-2 units)
// since the last rescale: P = 2^(s - m_ref) stays below 2^8; the algebra is exact.
constexpr float kRescaleSlack = 8.f;

// LDS stage layout: the latent parts of the 64 rows (1024 bytes each) at 0, the rotary parts
// (128 bytes each) at kRopeOff. 16-byte chunk c of latent row r sits at chunk c ^ lat_swz(r),
// chunk c of rotary row r at c ^ (r & 7). lat_swz is a bijection of r mod 16 that puts the two
// low row bits on chunk bits 2-3: 16 consecutive rows reading one chunk (the K reads of S) touch
// 16 distinct 16-byte bank slots, and so do 4 consecutive rows reading 4 consecutive chunks (the
// transposed V reads of 32 lanes); the rotary rows alternate bank halves already.
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }


constexpr int NW = 4;   // waves per workgroup
constexpr int kBR = 64; // query heads per unit

template <bool PAGED>
__global__ __launch_bounds__(256, 1) void decode_mla_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2][kTileBytes];
  // Exchange buffers, single: a step's values are read before the next step's first barrier and
  // rewritten only after it.
  __shared__ float sPmax[NW][32];                                  // partial row maxima
  __shared__ __attribute__((aligned(16))) bf16x8_t sP[NW][2][64];  // P of a key half
  __shared__ float sL[NW][32];                                        // row-sum halves

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int split = blockIdx.x;
  const int rb = blockIdx.y;
  const int b = blockIdx.z;
  const int g = 0;  // one latent KV head
  const int rg = wv & 1;  // row group: heads 32 rg .. of the unit
  const int kh = wv >> 1;  // key half of the scores and column half of O
  const int h0 = rb * kBR;
  const int my_h = h0 + rg * 32 + n;
  const bool row_ok = my_h < p.Hq && (rg * 32 + n) < p.block_r;
  const bool oth_ok = h0 + (rg ^ 1) * 32 + n < p.Hq && ((rg ^ 1) * 32 + n) < p.block_r;
  const bool bookkeeper = wv == 0 && lane == 0;  // counts and records the unit's tiles
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
  const int n_tiles = max(0, t_end - t_begin);
  // Contiguous cache: this sequence's rows; paged cache: the pool (the batch stride is then the
  // page stride) and this sequence's block-table row.
  const __bf16 *__restrict__ Kg = (const __bf16 *)p.k + (PAGED ? 0 : b * p.k_sb) + g * p.k_sh;
  const int32_t *__restrict__ bt = PAGED ? p.block_table + (int64_t)b * p.pages_per_seq : nullptr;
  // Paged: each lane holds the page of key `lane` of a tile (clamped to the sequence), loaded two
  // tiles ahead so the copies never wait on the table read; a row's page comes from the lane that
  // holds it through one cross-lane read.
  auto page_of_lane_key = [&](int tile) -> int {
    if constexpr (PAGED) {
      const int key = min(tile * kBlockC + lane, seq_len - 1);
      return bt[key >> p.page_shift];
    } else {
      return 0;
    }
  };
  const int64_t unit_tiles = ((int64_t)b * p.Hkv + g) * p.n_rblocks + rb;

  // Q fragments (B operand of S^T = K Q^T): query head my_h, columns 16 s + 8 hh .. + 7.
  bf16x8_t qf[kSteps];
  {
    const __bf16 *qrow = (const __bf16 *)p.q + b * p.q_sb + (int64_t)(row_ok ? my_h : 0) * p.q_sh;
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
      qf[s] = row_ok ? *(const bf16x8_t *)(qrow + 16 * s + 8 * hh) : (bf16x8_t)(__bf16)0.f;
    // Q is only ever an MFMA B operand, which may come from AGPRs: kept there, it leaves the
    // VGPRs to O^T and the K and V^T fragments read ahead of their MFMAs.
#pragma unroll
    for (int s = 0; s < kSteps; ++s) asm volatile("" : "+a"(qf[s]));
  }

  // Tile loads: wave load nn < 16 copies latent row i = wv + 4 nn (chunk L ^ lat_swz(i) of the
  // row from HBM to physical chunk L), loads 16 and 17 the rotary parts of rows 8 jr .. 8 jr + 7,
  // jr = wv + 4 (nn - 16) (lane L: row 8 jr + L / 8, logical chunk (L % 8) ^ (L / 8) to physical
  // L % 8). Rows past the end of the sequence copy its last row instead.
  auto issue_one = [&](int tile, int st, int nn, int pages) {
    const uint32_t lds_st = lds_addr(&smem[st][0]);
    if (nn < kRowLoads / NW) {
      const int i = wv + NW * nn;
      const int key = min(tile * kBlockC + i, seq_len - 1);  // wave-uniform
      const __bf16 *row;
      if constexpr (PAGED) {
        const int pg = __builtin_amdgcn_readlane(pages, key - tile * kBlockC);
        row = Kg + (int64_t)pg * p.k_sb + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.k_ss;
      } else {
        row = Kg + (int64_t)key * p.k_ss;
      }
      int ln = lane;  // opaque: recomputed per load instead of kept live across the MFMAs
      asm volatile("" : "+v"(ln));
      lds_dma16_s(row, (uint32_t)((ln ^ lat_swz(i)) << 4), lds_st + i * kLatBytes);
    } else {
      const int jr = wv + NW * (nn - kRowLoads / NW);
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int key = min(tile * kBlockC + 8 * jr + (ln >> 3), seq_len - 1);
      int64_t roff;
      if constexpr (PAGED) {
        const int pg = __shfl(pages, key - tile * kBlockC);  // all lanes take part
        roff = (int64_t)pg * p.k_sb + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.k_ss;
      } else {
        roff = (int64_t)key * p.k_ss;
      }
      const __bf16 *gp = Kg + roff + kDv + 8 * ((ln & 7) ^ (ln >> 3));
      lds_dma16(gp, lds_st + kRopeOff + jr * 1024);
    }
  };

  // Full tiles of a contiguous cache (no row past the sequence): latent row i of the tile sits
  // at a wave-uniform address (tile base + i rows), so a copy costs a 64-bit scalar add and the
  // lane's chunk offset, one of four per wave: i = wv + 4 nn has lat_swz(i) = 4 wv + nn % 4. The
  // rotary parts take a per-lane 32-bit offset from the tile base when 64 rows fit in 32 bits.
  const int64_t row_bytes = p.k_ss * 2;
  const bool off32 = !PAGED && row_bytes * kBlockC <= 0x7fffffffll;
  uint32_t lat_off[4], rope_voff[2];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) lat_off[q4] = (uint32_t)((lane ^ (4 * wv + q4)) << 4);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int jr = wv + NW * h2;
    rope_voff[h2] = (uint32_t)((8 * jr + (lane >> 3)) * row_bytes) + (uint32_t)kLatBytes +
                    (uint32_t)(16 * ((lane & 7) ^ (lane >> 3)));
  }
  // cur: this wave's next latent row (advanced by 4 rows per copy); tb: the tile's first row.
  auto issue_full = [&](const char *&cur, const char *tb, int st, int nn) {
    const uint32_t lds_st = lds_addr(&smem[st][0]);
    if (nn < kRowLoads / NW) {
      const int i = wv + NW * nn;
      lds_dma16_s(cur, lat_off[nn & 3], lds_st + i * kLatBytes);
      cur += NW * row_bytes;
    } else {
      const int h2 = nn - kRowLoads / NW;
      lds_dma16_s(tb, rope_voff[h2], lds_st + kRopeOff + (wv + NW * h2) * 1024);
    }
  };
  // Copy mode of the next tile: 0 none, 1 full contiguous tile, 2 any other.
  auto copy_mode = [&](int tile) -> int {
    if (tile < 0) return 0;
    return (off32 && (tile + 1) * kBlockC <= seq_len) ? 1 : 2;
  };

  // O^T of this wave's 128 columns for both row groups of the unit: oacc[r][db] holds columns
  // 128 wv + 32 db .. + 31 of heads 32 r .. + 31.
  f32x16_t oacc[2][kDvBlocks];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db) oacc[r][db] = (f32x16_t)0.f;
  float m_run = -INFINITY;    // running max of this wave's rows (base 2)
  float m_run_o = -INFINITY;  // running max of the other row group's rows (for the vote)
  float m_ref = -INFINITY, l_part = 0.f;
  float m_ref_o = -INFINITY;  // the other row group's reference max (for the rescale decision)
  unsigned visited = 0, skipped = 0;

  // S^T for this wave's 32 heads and its 32 keys (key half kh): A = K rows 32 kh + n of stage st,
  // B = the wave's query fragments; 36 k-steps, K fragments read KPF steps ahead. The next tile's
  // loads (next_tile >= 0) go out one per two k-steps between the MFMAs: each inline-asm load is
  // a scheduling boundary, so the reads and MFMAs between two loads stay in source order, and a
  // wave (alone on its SIMD) never stalls on a full load queue with its matrix core idle.
  // K reads of S: k-step s of this lane (row r = 32 kh + lane % 32, hb = lane / 32) reads
  // logical chunk 2 s + hb; for s < 32 that is physical chunk (2 s) ^ g, g = hb ^ lat_swz(r),
  // i.e. byte 256 (s / 8) + (32 (s % 8) ^ 16 g) of the row: eight per-lane offsets, computed
  // once; for s >= 32 the rotary chunk (2 (s - 32)) ^ (hb ^ (r & 7)).
  uint32_t s_off[8];
  uint32_t rope_off;
  {
    const int r = 32 * kh + (lane & 31), hb = lane >> 5;
    const uint32_t g16 = (uint32_t)((hb ^ lat_swz(r)) << 4);
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) s_off[b8] = (uint32_t)(r * kLatBytes) + ((32u * b8) ^ g16);
    rope_off = (uint32_t)(kRopeOff + r * kRopeBytes) | (uint32_t)((hb ^ (r & 7)) << 4);
  }
  auto compute_s = [&](auto mode_c, int st, int next_tile, int next_pages) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int KPF = 6;
    const char *tb = (const char *)(Kg + (int64_t)next_tile * kBlockC * p.k_ss);
    const char *cur = tb + (int64_t)wv * row_bytes;
    f32x16_t sacc = (f32x16_t)0.f;
    const char *sm = smem[st];
    const char *lat[8];
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) lat[b8] = sm + s_off[b8];
    auto rdk = [&](int s2) {
      return s2 < kLatSteps ? *(const bf16x8_t *)(lat[s2 & 7] + 256 * (s2 >> 3))
                            : *(const bf16x8_t *)(sm + (rope_off ^ (32u * (s2 - kLatSteps))));
    };
    bf16x8_t fr[kSteps];
#pragma unroll
    for (int s2 = 0; s2 < KPF; ++s2) fr[s2] = rdk(s2);
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      if (s2 + KPF < kSteps) fr[s2 + KPF] = rdk(s2 + KPF);
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s2], qf[s2], sacc, 0, 0, 0);
      if constexpr (MODE == 1) {
        if (s2 & 1) issue_full(cur, tb, st ^ 1, s2 >> 1);
      } else if constexpr (MODE == 2) {
        if (s2 & 1) issue_one(next_tile, st ^ 1, s2 >> 1, next_pages);
      }
      // Without this the scheduler sinks the K reads next to their MFMAs to save registers,
      // and each MFMA waits out an LDS read latency.
      __builtin_amdgcn_sched_barrier(0);
    }
    return sacc;
  };

  // Score (key) of accumulator element i: 32 kh + 8 (i / 4) + 4 hh + i % 4 within the tile.
  // Keys past the end and (window) keys before the first visible one score -inf.
  auto mask_tile = [&](int tile, f32x16_t &sacc) {
    const int k0 = tile * kBlockC + 32 * kh;
    if (k0 + 32 > seq_len || k0 < first_key) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= seq_len || key < first_key) sacc[i] = -INFINITY;
      }
    }
  };

  // Row test for one row: margin exactly 0 at a new row maximum (mt2 rounded on its own, no
  // fused multiply-add); returns keep and advances the running max.
  auto row_test = [&](float tmax, float &mr, bool ok, float &margin) {
    const float mt2 = __fmul_rn(tmax, p.scale_log2);
    const float delta = (mt2 >= mr) ? 0.f : __fsub_rn(mt2, mr);
    mr = fmaxf(mr, mt2);
    const bool valid = ok && mt2 > -INFINITY;
    margin = valid ? delta : -INFINITY;
    return valid && !(delta < p.tau_log2);
  };


  // O^T (this wave's 128 columns, both row groups) += V^T P^T over the tile's 64 keys: k-step ks
  // (keys 16 ks .. 16 ks + 15) takes as B the bf16 P fragments of those keys for row groups 0 and
  // 1, as published by waves 2 (ks / 2) and 2 (ks / 2) + 1, and as A 4 column blocks of V^T
  // (transpose reads of the row-major tile, stage st), each read once, RA reads ahead (held there
  // by a scheduling barrier per fragment), for two MFMAs. The read of column block db, rows 16 ks + vrow (and + 8) is at a per-lane offset plus
  // 16384 ks: with f = lat_swz(vrow), chunk 16 w + 4 db + vcb sits at 16 w + ((4 db + vcb) ^ f),
  // and the row + 8 at f ^ 2.
  uint32_t v_off[kDvBlocks], v_off_hi[kDvBlocks];
  {
    const int vrow = 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int vcb = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int f = lat_swz(vrow);
#pragma unroll
    for (int db = 0; db < kDvBlocks; ++db) {
      const uint32_t base = (uint32_t)(vrow * kLatBytes + 8 * (lane & 1) + 16 * 16 * wv);
      v_off[db] = base + 16u * (uint32_t)((4 * db + vcb) ^ f);
      v_off_hi[db] = base + 8u * kLatBytes + 16u * (uint32_t)((4 * db + vcb) ^ f ^ 2);
    }
  }
  auto pv = [&](int st) {
    constexpr int NM = 4 * kDvBlocks;  // 16 V^T fragments: (ks, db) = (m / 4, m % 4)
    constexpr int RA = 3;
    // B operands: P of row group r, k-step ks, as published by wave r + 2 (ks / 2).
    bf16x8_t pb[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) pb[r][ks] = sP[r + 2 * (ks >> 1)][ks & 1][lane];
    const char *vl = smem[st];
    auto rdv = [&](int m) {
      const int ks = m / kDvBlocks, db = m % kDvBlocks;
      const char *p0 = vl + v_off[db] + 16 * kLatBytes * ks;
      const char *p1 = vl + v_off_hi[db] + 16 * kLatBytes * ks;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t va[RA + 1];
#pragma unroll
    for (int m = 0; m < RA; ++m) va[m] = rdv(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + RA < NM) va[(m + RA) % (RA + 1)] = rdv(m + RA);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        oacc[r][m % kDvBlocks] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            va[m % (RA + 1)], pb[r][m / kDvBlocks], oacc[r][m % kDvBlocks], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // P = 2^(s - m_ref) of this wave's rows and key half in bf16, published in sP for every wave's
  // P.V; returns the lane's part of the row sums of the rounded P.
  const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
  auto make_p = [&](const f32x16_t &sacc) {
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      bf16x8_t pk;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pk[e] = (__bf16)exp2_fast(fmaf(sacc[8 * h2 + e], p.scale_log2, -m_use));
      const bf16x2_t x0 = {pk[0], pk[1]}, x1 = {pk[2], pk[3]};
      const bf16x2_t x2 = {pk[4], pk[5]}, x3 = {pk[6], pk[7]};
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(x0, one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(x1, one, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(x2, one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(x3, one, ps1, false);
      sP[wv][h2][lane] = pk;
    }
    return ps0 + ps1;
  };

  // Two barriers per tile: (1) tile j is in LDS, the other stage is free; (2) every wave's
  // partial row maxima and its bf16 P (formed with the current reference max before the test)
  // are visible -- each wave then takes the test for all 64 rows of the unit, so the decision
  // needs no vote exchange. A kept tile that moves the reference max forms P again and
  // publishes it behind a third barrier.
  // Paged: `ahead` is the table read of the tile after next; it is taken over (as the pages of
  // the next tile's copies) only after the wait at the top of the following step.
  int ahead = 0;
  if (n_tiles > 0) {
    const int pages0 = page_of_lane_key(t_begin);
    if constexpr (PAGED) __builtin_amdgcn_s_waitcnt(0);  // table read landed before any copy
#pragma unroll
    for (int nn = 0; nn < kLoadsPerTile / NW; ++nn) issue_one(t_begin, 0, nn, pages0);
    if (n_tiles > 1) ahead = page_of_lane_key(t_begin + 1);
  }
  for (int j = 0; j < n_tiles; ++j) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int pages_next = ahead;  // landed: the wait above drained every load
    if (PAGED && j + 2 < n_tiles) ahead = page_of_lane_key(t_begin + j + 2);
    const int nt = j + 1 < n_tiles ? t_begin + j + 1 : -1;
    const int cm = copy_mode(nt);
    f32x16_t sacc;
    if (cm == 1)
      sacc = compute_s(std::integral_constant<int, 1>{}, j & 1, nt, pages_next);
    else if (cm == 2)
      sacc = compute_s(std::integral_constant<int, 2>{}, j & 1, nt, pages_next);
    else
      sacc = compute_s(std::integral_constant<int, 0>{}, j & 1, nt, pages_next);
    mask_tile(t_begin + j, sacc);
    {
      float m[6];
#pragma unroll
      for (int i = 0; i < 5; ++i) m[i] = max3f(sacc[3 * i], sacc[3 * i + 1], sacc[3 * i + 2]);
      m[5] = sacc[15];
      const float pm = max_halves(max3f(max3f(m[0], m[1], m[2]), max3f(m[3], m[4], m[5]), m[5]));
      if (hh == 0) sPmax[wv][n] = pm;
    }
    // P of this wave's rows and key half with the current reference max, published before the
    // test: when the tile is kept and needs no rescale, the partner's half is already visible
    // after the next barrier.
    float ps = make_p(sacc);
    __syncthreads();
    float mg_own, mg_oth;
    const bool keep_own =
        row_test(fmaxf(sPmax[wv][n], sPmax[wv ^ 2][n]), m_run, row_ok, mg_own);
    const bool keep_oth = row_test(fmaxf(sPmax[wv ^ 1][n], sPmax[wv ^ 3][n]),
                                   m_run_o, oth_ok, mg_oth);
    const bool keep = __ballot(keep_own || keep_oth) != 0ull;
    if (p.tile_margin) {
      float dm = fmaxf(mg_own, mg_oth);
      asm volatile("" : "+v"(dm));  // keeps the reduction inside the branch
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dm = fmaxf(dm, __shfl_xor(dm, o));
      if (bookkeeper) p.tile_margin[unit_tiles * p.n_tiles + t_begin + j] = dm * kLn2;
    }
    if (bookkeeper) {
      ++visited;
      skipped += keep ? 0u : 1u;
      if (p.tile_status) p.tile_status[unit_tiles * p.n_tiles + t_begin + j] = keep ? 0 : 1;
    }
    if (keep) {
      // Rescale when some row of the unit has outgrown its reference max by more than the
      // slack; every wave sees all 64 rows' maxima, so the decision (and the barrier in it) is
      // the same in every wave. The first kept tile of a split always takes it.
      if (__ballot(m_run > m_ref + kRescaleSlack || m_run_o > m_ref_o + kRescaleSlack) != 0ull) {
        const float alpha = exp2_fast(m_ref - ((m_run == -INFINITY) ? 0.f : m_run));
        const float alpha_o = exp2_fast(m_ref_o - ((m_run_o == -INFINITY) ? 0.f : m_run_o));
        l_part *= alpha;
        const float a0 = rg == 0 ? alpha : alpha_o, a1 = rg == 0 ? alpha_o : alpha;
#pragma unroll
        for (int db = 0; db < kDvBlocks; ++db) {
          oacc[0][db] *= a0;
          oacc[1][db] *= a1;
        }
        m_ref = m_run;
        m_ref_o = m_run_o;
        ps = make_p(sacc);
        __syncthreads();
      }
      l_part += ps;
      pv(j & 1);
    }
  }

  // Epilogue: the row sum of a row group is split over the key halves of its two waves (both
  // scaled to the same m_ref); normalised O (this wave's 128 columns of all 64 rows) or the
  // split's partial, and LSE.
  const float l_mine = sum_halves(l_part);
  if (hh == 0) sL[wv][n] = l_mine;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int h = h0 + 32 * r + n;
    if (!(h < p.Hq && 32 * r + n < p.block_r)) continue;
    const float l_tot = sL[r][n] + sL[r + 2][n];
    const float m_r = r == rg ? m_ref : m_ref_o;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (p.num_splits == 1) {
      __bf16 *orow = (__bf16 *)p.o + b * p.o_sb + (int64_t)h * p.o_sh + 128 * wv;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = db * 32 + 8 * ig + 4 * hh;
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          const f32x16_t &oa = oacc[r][db];
          bf16x4_t ov = {(__bf16)(oa[4 * ig + 0] * inv), (__bf16)(oa[4 * ig + 1] * inv),
                         (__bf16)(oa[4 * ig + 2] * inv), (__bf16)(oa[4 * ig + 3] * inv)};
          *(bf16x4_t *)(orow + d0) = ov;
        }
      }
      if (p.lse && hh == 0 && wv == 0)
        p.lse[(int64_t)b * p.Hq + h] = l_tot > 0.f ? (m_r + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t row = ((int64_t)b * p.Hq + h) * p.num_splits + split;
      float *op = p.o_part + row * kDv + 128 * wv;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = db * 32 + 8 * ig + 4 * hh;
          const f32x16_t &oa = oacc[r][db];
          *(float4 *)(op + d0) = make_float4(oa[4 * ig + 0] * inv, oa[4 * ig + 1] * inv,
                                             oa[4 * ig + 2] * inv, oa[4 * ig + 3] * inv);
        }
      }
      if (hh == 0 && wv == 0) p.lse_part[row] = l_tot > 0.f ? m_r + __log2f(l_tot) : -INFINITY;
    }
  }
  if (bookkeeper) {
    if (p.counters && visited) {
      atomicAdd(&p.counters[0], (unsigned long long)visited);
      atomicAdd(&p.counters[1], (unsigned long long)skipped);
    }
    if (p.tile_status || p.tile_margin) {
      // Not visited: the rest of this split's range past the sequence; with a window, split 0
      // also marks the tiles before it and the last split those after every split's range.
      const int cover_end = min(t_base + p.num_splits * p.tiles_per_split, p.n_tiles);
      for (int t = 0; t < p.n_tiles; ++t) {
        const bool mine = (t >= t_begin + n_tiles && t < t_split_end) ||
                          (split == 0 && t < t_base) ||
                          (split == p.num_splits - 1 && t >= cover_end);
        if (!mine) continue;
        if (p.tile_status) p.tile_status[unit_tiles * p.n_tiles + t] = 2;
        if (p.tile_margin) p.tile_margin[unit_tiles * p.n_tiles + t] = -INFINITY;
      }
    }
  }
}

}  // namespace

hipError_t launch_decode_mla(const DecodeParams &p, hipStream_t stream) {
  if (p.block_r > kBR) return hipErrorInvalidValue;
  const dim3 grid(p.num_splits, p.n_rblocks, p.B);
  if (p.block_table)
    hipLaunchKernelGGL(decode_mla_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_mla_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace blasst

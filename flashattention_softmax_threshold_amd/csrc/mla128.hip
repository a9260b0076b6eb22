// mla128.hip -- MLA-shaped BLASST decode on gfx950 with every query head of the latent KV head
// in one unit (B_r = 128): d_qk = 576, V is the first 512 columns of K.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm": per key tile, skip the softmax
// and P.V when tile_max - running_max < ln(lambda) for every query row of the tile. The BLASST
// talk notes ("kernel design") observe that MLA decode can be compute-bound, so skipping the P.V
// work pays there even though V costs no extra traffic: the V tile is the K tile already on chip.
//
// Work unit (one workgroup of 4 waves, one wave per SIMD): (sequence b, block of up to 128 heads,
// split of the key range). Wave w owns query heads 32 w .. 32 w + 31 of the block outright: it
// scores them against all 64 keys of a tile and accumulates their whole output row, so the row
// maxima, the rescale and P never leave the wave. Per key tile of 64 keys:
//   * the K tile (64 x 576 bf16, 72 KB) goes from HBM straight into LDS (global_load_lds_dwordx4,
//     two stages), copied once for all 128 heads; the next tile's copies are issued between the
//     MFMAs of this tile's scores;
//   * S^T (64 keys x 32 heads) = K Q^T with v_mfma_f32_32x32x16_bf16: two 32-key blocks over 36
//     k-steps, A = K rows from LDS, B = the wave's query fragments held in registers;
//   * each wave tests its 32 rows and publishes one vote word; after a barrier every wave ORs the
//     four words, so all reach the same decision;
//   * a kept tile: P = exp2(S - m_ref) in bf16 stays in the score registers, which already hold
//     the B operand layout of O^T (512 x 32) += V^T P^T; V^T is read from the same LDS tile with
//     ds_read_b64_tr_b16. O^T (256 registers a wave) lives in the accumulation registers.
// Against the 64-head kernel (mla.hip) every K tile is copied to LDS once instead of twice and
// the two exchange barriers of the unit's P and maxima are gone; each V^T fragment feeds one
// MFMA instead of two.
// LDS stage layout, swizzles and copy pattern are those of mla.hip: the latent parts of a tile's
// rows (64 x 1024 bytes) and their rotary parts (64 x 128 bytes) apart, 16-byte chunks
// XOR-swizzled by the row so that the K and V^T reads are conflict-free.
// Splits write normalised partial O and base-2 LSE to the workspace; the split merge combines.
#include "internal.h"
#include "lds_dma.h"
#include "mla128_agpr.h"

#include <math.h>

#include <type_traits>
#include <utility>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
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
constexpr int kCB = kDv / 32;                       // 16 output column blocks of 32
constexpr int NW = 4;                               // waves per workgroup
constexpr int kBR = 128;                            // query heads per unit
// O and l are rescaled only when some row's max has grown by more than this (base-2 units)
// since the last rescale: P = 2^(s - m_ref) stays below 2^8; the algebra is exact.
constexpr float kRescaleSlack = 8.f;
// LDS read-ahead: K fragments of the scores 2 k-steps (4 fragments) ahead, V^T fragments of P.V
// 4 MFMAs ahead (deeper read-ahead measured no faster; 3 k-steps makes the paged instance spill).
constexpr int kKpf = 2;
constexpr int kRa = 4;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }
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
// Chunk swizzle of latent row r: a bijection of r mod 16 that puts the two low row bits on chunk
// bits 2-3 (16 rows reading one chunk, or 4 rows reading 4 consecutive chunks, hit 16 distinct
// 16-byte bank slots).
__device__ __forceinline__ int lat_swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// O^T block cb (a[16 cb : 16 cb + 15]) through the statements of mla128_agpr.h; cb is a constant
// wherever these are called (unrolled loops), so each switch folds to one statement.
#define BLASST_AGPR_CASES(F, ...)                                                              \
  switch (cb) {                                                                                \
    case 0: agpr::F<0>(__VA_ARGS__); break;   case 1: agpr::F<1>(__VA_ARGS__); break;          \
    case 2: agpr::F<2>(__VA_ARGS__); break;   case 3: agpr::F<3>(__VA_ARGS__); break;          \
    case 4: agpr::F<4>(__VA_ARGS__); break;   case 5: agpr::F<5>(__VA_ARGS__); break;          \
    case 6: agpr::F<6>(__VA_ARGS__); break;   case 7: agpr::F<7>(__VA_ARGS__); break;          \
    case 8: agpr::F<8>(__VA_ARGS__); break;   case 9: agpr::F<9>(__VA_ARGS__); break;          \
    case 10: agpr::F<10>(__VA_ARGS__); break; case 11: agpr::F<11>(__VA_ARGS__); break;        \
    case 12: agpr::F<12>(__VA_ARGS__); break; case 13: agpr::F<13>(__VA_ARGS__); break;        \
    case 14: agpr::F<14>(__VA_ARGS__); break; default: agpr::F<15>(__VA_ARGS__); break;        \
  }
__device__ __forceinline__ void o_mfma(int cb, const bf16x8_t &a, const bf16x8_t &b) {
  BLASST_AGPR_CASES(mfma, a, b)
}
__device__ __forceinline__ void o_scale(int cb, float alpha) { BLASST_AGPR_CASES(scale, alpha) }
__device__ __forceinline__ void o_read(int cb, float (&x)[16]) { BLASST_AGPR_CASES(read, x) }
#undef BLASST_AGPR_CASES

// f(std::integral_constant<int, I>) for I = 0 .. N - 1, in order: indices that must be
// compile-time constants (register blocks, array slots) whatever the unroller decides.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <bool PAGED>
__global__ __launch_bounds__(256, 1) void decode_mla128_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2][kTileBytes];
  // A tile's votes and margins: written after the step's first barrier, read after its second.
  __shared__ int sVote[NW];
  __shared__ float sMarg[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int split = blockIdx.x;
  const int rb = blockIdx.y;
  const int b = blockIdx.z;
  const int g = 0;  // one latent KV head
  const int row = 32 * wv + n;  // this lane's row of the unit
  const int my_h = rb * p.block_r + row;
  const bool row_ok = row < p.block_r && my_h < p.Hq;
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
  const __bf16 *__restrict__ Kg = (const __bf16 *)p.k + (PAGED ? 0 : b * p.k_sb) + g * p.k_sh;
  const int32_t *__restrict__ bt = PAGED ? p.block_table + (int64_t)b * p.pages_per_seq : nullptr;
  // Paged: each lane holds the page of key `lane` of a tile (clamped to the sequence), loaded two
  // tiles ahead so the copies never wait on the table read.
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
  }

  // Tile copies: wave load nn < 16 copies latent row i = wv + 4 nn (chunk L ^ lat_swz(i) of the
  // row from HBM to physical chunk L), loads 16 and 17 the rotary parts of rows 8 jr .. 8 jr + 7,
  // jr = wv + 4 (nn - 16) (lane L: row 8 jr + L / 8, logical chunk (L % 8) ^ (L / 8) to physical
  // L % 8). Rows past the end of the sequence copy its last row instead.
  auto issue_one = [&](int tile, int st, int nn, int pages) {
    const uint32_t lds_st = lds_addr(&smem[st][0]);
    if (nn < kRowLoads / NW) {
      const int i = wv + NW * nn;
      const int key = min(tile * kBlockC + i, seq_len - 1);  // wave-uniform
      const __bf16 *rowp;
      if constexpr (PAGED) {
        const int pg = __builtin_amdgcn_readlane(pages, key - tile * kBlockC);
        rowp = Kg + (int64_t)pg * p.k_sb + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.k_ss;
      } else {
        rowp = Kg + (int64_t)key * p.k_ss;
      }
      int ln = lane;  // opaque: recomputed per load instead of kept live across the MFMAs
      asm volatile("" : "+v"(ln));
      lds_dma16_s(rowp, (uint32_t)((ln ^ lat_swz(i)) << 4), lds_st + i * kLatBytes);
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
  // Full tiles of a contiguous cache (no row past the sequence): latent row i sits at a
  // wave-uniform address (tile base + i rows), so a copy costs a 64-bit scalar add and one of the
  // wave's four chunk offsets (i = wv + 4 nn has lat_swz(i) = 4 wv + nn % 4); the rotary parts
  // take a per-lane 32-bit offset from the tile base when 64 rows fit in 32 bits.
  // The per-lane offsets are recomputed per copy from an opaque lane index (two or three
  // vector instructions) rather than held in registers across the scores.
  const int64_t row_bytes = p.k_ss * 2;
  const bool off32 = !PAGED && row_bytes * kBlockC <= 0x7fffffffll;
  auto issue_full = [&](const char *&cur, const char *tb, int st, int nn) {
    const uint32_t lds_st = lds_addr(&smem[st][0]);
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (nn < kRowLoads / NW) {
      const int i = wv + NW * nn;
      lds_dma16_s(cur, (uint32_t)((ln ^ (4 * wv + (nn & 3))) << 4), lds_st + i * kLatBytes);
      cur += NW * row_bytes;
    } else {
      const int jr = wv + NW * (nn - kRowLoads / NW);
      const uint32_t voff = (uint32_t)((8 * jr + (ln >> 3)) * (uint32_t)row_bytes) +
                            (uint32_t)kLatBytes + (uint32_t)(16 * ((ln & 7) ^ (ln >> 3)));
      lds_dma16_s(tb, voff, lds_st + kRopeOff + jr * 1024);
    }
  };
  // Copy mode of the next tile: 0 none, 1 full contiguous tile, 2 any other.
  auto copy_mode = [&](int tile) -> int {
    if (tile < 0) return 0;
    return (off32 && (tile + 1) * kBlockC <= seq_len) ? 1 : 2;
  };

  // O^T of this wave's 32 heads: block cb (a[16 cb : 16 cb + 15]) holds columns 32 cb .. + 31.
  agpr::zero_all();
  float m_run = -INFINITY;  // running max of this lane's row (base 2)
  float m_ref = -INFINITY, l_part = 0.f;
  unsigned visited = 0, skipped = 0;

  // K reads of S: k-step s of this lane (row r = 32 kb + lane % 32 of key block kb) reads logical
  // chunk 2 s + hh; for s < 32 that is byte 256 (s / 8) + (32 (s % 8) ^ 16 (hh ^ lat_swz(r))) of
  // the latent row (eight per-lane offsets, computed once; key block 1 is 32 rows = 32 KiB on),
  // for s >= 32 the rotary chunk (2 (s - 32)) ^ (hh ^ (r & 7)) (key block 1: 4 KiB on).
  uint32_t s_off[8];
  uint32_t rope_off;
  {
    const int r = n;
    const uint32_t g16 = (uint32_t)((hh ^ lat_swz(r)) << 4);
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) s_off[b8] = (uint32_t)(r * kLatBytes) + ((32u * b8) ^ g16);
    rope_off = (uint32_t)(kRopeOff + r * kRopeBytes) | (uint32_t)((hh ^ (r & 7)) << 4);
  }
  // S^T of the wave's 32 heads against the 64 keys of stage st: k-step s issues the MFMAs of
  // both key blocks with the same Q fragment; K fragments read KPF k-steps ahead. The next tile's
  // copies go out one per two k-steps; each inline-asm copy and the scheduling barrier per step
  // keep the reads and MFMAs in source order.
  auto compute_s = [&](auto mode_c, int st, int next_tile, int next_pages, f32x16_t &s0,
                       f32x16_t &s1) {
    constexpr int MODE = decltype(mode_c)::value;
    constexpr int KPF = kKpf;
    const char *tb = (const char *)(Kg + (int64_t)next_tile * kBlockC * p.k_ss);
    const char *cur = tb + (int64_t)wv * row_bytes;
    s0 = (f32x16_t)0.f;
    s1 = (f32x16_t)0.f;
    const char *sm = smem[st];
    const char *lat[8];
#pragma unroll
    for (int b8 = 0; b8 < 8; ++b8) lat[b8] = sm + s_off[b8];
    auto rdk = [&](int s2, int kb) {
      return s2 < kLatSteps
                 ? *(const bf16x8_t *)(lat[s2 & 7] + 256 * (s2 >> 3) + 32768 * kb)
                 : *(const bf16x8_t *)(sm + (rope_off ^ (32u * (s2 - kLatSteps))) + 4096 * kb);
    };
    bf16x8_t fr[kSteps][2];
#pragma unroll
    for (int s2 = 0; s2 < KPF; ++s2) {
      fr[s2][0] = rdk(s2, 0);
      fr[s2][1] = rdk(s2, 1);
    }
#pragma unroll
    for (int s2 = 0; s2 < kSteps; ++s2) {
      if (s2 + KPF < kSteps) fr[s2 + KPF][0] = rdk(s2 + KPF, 0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s2][0], qf[s2], s0, 0, 0, 0);
      if (s2 + KPF < kSteps) fr[s2 + KPF][1] = rdk(s2 + KPF, 1);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s2][1], qf[s2], s1, 0, 0, 0);
      if constexpr (MODE == 1) {
        if (s2 & 1) issue_full(cur, tb, st ^ 1, s2 >> 1);
      } else if constexpr (MODE == 2) {
        if (s2 & 1) issue_one(next_tile, st ^ 1, s2 >> 1, next_pages);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Key of accumulator element i of key block kb: 32 kb + 8 (i / 4) + 4 hh + i % 4 in the tile.
  // Keys past the end and (window) keys before the first visible one score -inf.
  auto mask_block = [&](int tile, int kb, f32x16_t &sacc) {
    const int k0 = tile * kBlockC + 32 * kb;
    if (k0 + 32 > seq_len || k0 < first_key) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= seq_len || key < first_key) sacc[i] = -INFINITY;
      }
    }
  };

  // V^T reads of P.V: the A operand of k-step ks (keys 16 ks ..) and column block cb is two
  // transposed reads, rows 16 ks + vrow and + 8; with f = lat_swz(vrow), chunk 4 cb + vcb of the
  // latent row sits at 16 (cb / 4) + ((4 (cb % 4) + vcb) ^ f), and the row + 8 at f ^ 2. Four
  // per-lane offsets each; cb / 4 and ks are constant offsets.
  // O^T += V^T P^T over the tile's 64 keys, with P formed on the way. P = 2^(s - m_ref) in bf16
  // of k-step ks is the B operand of that k-step: score registers 8 (ks % 2) .. + 7 of key block
  // ks / 2, this lane's keys 16 ks + 8 (e / 4) + 4 hh + e % 4 -- the same keys the transposed V
  // reads give its A rows. P of k-step 0 is formed first; P of k-step ks + 1 one element per MFMA
  // slot between the 16 MFMAs of k-step ks (the exponentials run while the matrix pipe works).
  // The A operand of k-step ks and column block cb is two transposed reads, rows 16 ks + vrow and
  // + 8; with f = lat_swz(vrow), chunk 4 cb + vcb of the latent row sits at
  // 16 (cb / 4) + ((4 (cb % 4) + vcb) ^ f), and the row + 8 at f ^ 2: four per-lane offsets
  // each, cb / 4 and ks constant offsets. Returns this lane's part of the row sum of the rounded
  // P.
  const bf16x2_t one = {(__bf16)1.f, (__bf16)1.f};
  auto pv = [&](int st, const f32x16_t &s0, const f32x16_t &s1) {
    constexpr int NM = 4 * kCB;  // (ks, cb) = (m / 16, m % 16)
    constexpr int RA = kRa;
    const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
    auto p_elem = [&](int ks, int e) {
      const f32x16_t &sa = (ks < 2) ? s0 : s1;
      return exp2_fast(fmaf(sa[8 * (ks & 1) + e], p.scale_log2, -m_use));
    };
    float ps0 = 0.f, ps1 = 0.f;
    // Rounds 8 elements to a bf16 B operand and adds them (as rounded) to the row sums.
    auto pack = [&](const float (&x)[8]) {
      bf16x8_t pk;
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = (__bf16)x[e];
      const bf16x2_t x0 = {pk[0], pk[1]}, x1 = {pk[2], pk[3]};
      const bf16x2_t x2 = {pk[4], pk[5]}, x3 = {pk[6], pk[7]};
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(x0, one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(x1, one, ps1, false);
      ps0 = __builtin_amdgcn_fdot2_f32_bf16(x2, one, ps0, false);
      ps1 = __builtin_amdgcn_fdot2_f32_bf16(x3, one, ps1, false);
      return pk;
    };
    const char *vl = smem[st];
    // V^T read offsets of this lane, formed here so that they are not held across the scores.
    uint32_t v_off[4], v_off_hi[4];
    {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int vrow = 4 * (ln >> 5) + ((ln & 15) >> 2);
      const int vcb = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
      const int f = lat_swz(vrow);
      const uint32_t base = (uint32_t)(vrow * kLatBytes + 8 * (ln & 1));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        v_off[db] = base + 16u * (uint32_t)((4 * db + vcb) ^ f);
        v_off_hi[db] = base + 8u * kLatBytes + 16u * (uint32_t)((4 * db + vcb) ^ f ^ 2);
      }
    }
    auto rdv = [&](int m) {
      const int ks = m / kCB, cb = m % kCB;
      const char *p0 = vl + v_off[cb & 3] + 256 * (cb >> 2) + 16 * kLatBytes * ks;
      const char *p1 = vl + v_off_hi[cb & 3] + 256 * (cb >> 2) + 16 * kLatBytes * ks;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
      const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8_t va[RA + 1];
#pragma unroll
    for (int m = 0; m < RA; ++m) va[m] = rdv(m);
    bf16x8_t pb[4];
    {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = p_elem(0, e);
      pb[0] = pack(x);
    }
    float xn[8];
    static_for<NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      constexpr int ks = m / kCB, cb = m % kCB;
      if constexpr (m + RA < NM) va[(m + RA) % (RA + 1)] = rdv(m + RA);
      agpr::mfma<cb>(va[m % (RA + 1)], pb[ks]);
      if constexpr (ks < 3) {
        if constexpr (cb < 8) xn[cb] = p_elem(ks + 1, cb);
        if constexpr (cb == 8) pb[ks + 1] = pack(xn);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    return ps0 + ps1;
  };

  // Two barriers per tile: (1) tile j is in LDS and every wave is done with tile j - 1, so its
  // stage may take tile j + 1; (2) the four vote words of tile j are visible.
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
    f32x16_t s0, s1;
    if (cm == 1)
      compute_s(std::integral_constant<int, 1>{}, j & 1, nt, pages_next, s0, s1);
    else if (cm == 2)
      compute_s(std::integral_constant<int, 2>{}, j & 1, nt, pages_next, s0, s1);
    else
      compute_s(std::integral_constant<int, 0>{}, j & 1, nt, pages_next, s0, s1);
    mask_block(t_begin + j, 0, s0);
    mask_block(t_begin + j, 1, s1);
    // Row test: the tile max of this lane's row (its 32 keys, then the other half-wave's), the
    // margin exactly 0 at a new row maximum (mt2 rounded on its own, no fused multiply-add).
    float mg;
    bool keep_row;
    {
      float m[11];
#pragma unroll
      for (int i = 0; i < 5; ++i) m[i] = max3f(s0[3 * i], s0[3 * i + 1], s0[3 * i + 2]);
#pragma unroll
      for (int i = 0; i < 5; ++i) m[5 + i] = max3f(s1[3 * i], s1[3 * i + 1], s1[3 * i + 2]);
      m[10] = fmaxf(s0[15], s1[15]);
      const float tmax = max_halves(max3f(max3f(m[0], m[1], m[2]), max3f(m[3], m[4], m[5]),
                                          max3f(max3f(m[6], m[7], m[8]), m[9], m[10])));
      const float mt2 = __fmul_rn(tmax, p.scale_log2);
      const float delta = (mt2 >= m_run) ? 0.f : __fsub_rn(mt2, m_run);
      m_run = fmaxf(m_run, mt2);
      const bool valid = row_ok && mt2 > -INFINITY;
      mg = valid ? delta : -INFINITY;
      keep_row = valid && !(delta < p.tau_log2);
    }
    const bool vote = __ballot(keep_row) != 0ull;
    if (lane == 0) sVote[wv] = vote ? 1 : 0;
    if (p.tile_margin) {
      float dm = mg;
      asm volatile("" : "+v"(dm));  // keeps the reduction inside the branch
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dm = fmaxf(dm, __shfl_xor(dm, o));
      if (lane == 0) sMarg[wv] = dm;
    }
    __syncthreads();
    const bool keep = (sVote[0] | sVote[1] | sVote[2] | sVote[3]) != 0;
    if (bookkeeper) {
      ++visited;
      skipped += keep ? 0u : 1u;
      if (p.tile_status) p.tile_status[unit_tiles * p.n_tiles + t_begin + j] = keep ? 0 : 1;
      if (p.tile_margin)
        p.tile_margin[unit_tiles * p.n_tiles + t_begin + j] =
            fmaxf(fmaxf(sMarg[0], sMarg[1]), fmaxf(sMarg[2], sMarg[3])) * kLn2;
    }
    if (keep) {
      // The wave's rows are its own: it rescales them alone, when one of them has outgrown its
      // reference max by more than the slack. The first kept tile of a split always does.
      if (__ballot(m_run > m_ref + kRescaleSlack) != 0ull) {
        const float alpha = exp2_fast(m_ref - ((m_run == -INFINITY) ? 0.f : m_run));
        l_part *= alpha;
        agpr::settle();
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) o_scale(cb, alpha);
        m_ref = m_run;
      }
      l_part += pv(j & 1, s0, s1);
    }
  }

  // Epilogue: the two half-waves hold the row sums of different keys of the same row (both
  // scaled to the same m_ref); normalised O of the wave's 32 heads, or the split's partial, and
  // LSE.
  const float l_tot = sum_halves(l_part);
  agpr::settle();
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (p.num_splits == 1) {
      __bf16 *orow = (__bf16 *)p.o + b * p.o_sb + (int64_t)my_h * p.o_sh;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        float oa[16];
        o_read(cb, oa);
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = cb * 32 + 8 * ig + 4 * hh;
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          bf16x4_t ov = {(__bf16)(oa[4 * ig + 0] * inv), (__bf16)(oa[4 * ig + 1] * inv),
                         (__bf16)(oa[4 * ig + 2] * inv), (__bf16)(oa[4 * ig + 3] * inv)};
          *(bf16x4_t *)(orow + d0) = ov;
        }
      }
      if (p.lse && hh == 0)
        p.lse[(int64_t)b * p.Hq + my_h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = ((int64_t)b * p.Hq + my_h) * p.num_splits + split;
      float *op = p.o_part + prow * kDv;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        float oa[16];
        o_read(cb, oa);
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = cb * 32 + 8 * ig + 4 * hh;
          *(float4 *)(op + d0) = make_float4(oa[4 * ig + 0] * inv, oa[4 * ig + 1] * inv,
                                             oa[4 * ig + 2] * inv, oa[4 * ig + 3] * inv);
        }
      }
      if (hh == 0) p.lse_part[prow] = l_tot > 0.f ? m_ref + __log2f(l_tot) : -INFINITY;
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

hipError_t launch_decode_mla128(const DecodeParams &p, hipStream_t stream) {
  if (p.block_r > kBR) return hipErrorInvalidValue;
  const dim3 grid(p.num_splits, p.n_rblocks, p.B);
  if (p.block_table)
    hipLaunchKernelGGL(decode_mla128_kernel<true>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_mla128_kernel<false>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace blasst

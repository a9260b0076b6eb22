// mla.hip -- MLA-shaped BLASST decode on gfx950: many query heads share one latent KV head,
// d_qk = 576, and V is the first 512 columns of K.
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm": per key tile, skip the softmax
// and P.V when tile_max - running_max < ln(lambda) for every query row of the tile. The BLASST
// talk notes ("kernel design") observe that MLA decode can be compute-bound, so skipping the P.V
// work pays there even though V costs no extra traffic: the V tile is the K tile already on chip.
//
// Work unit (one workgroup of 4 waves): (sequence b, block of B_r = 64 heads, split of the key
// range). Wave w owns query heads 32 (w % 2) .. + 31 of the block and output columns
// 256 (w / 2) .. + 255: both waves of a head pair form the same scores (the Q K^T work is done
// twice) so that each needs only half of O in accumulation registers -- 32 rows x 512 columns of
// fp32 plus the score tile would not fit the 256 accumulation registers of a wave. Per key tile
// of 64 keys:
//   * the K tile (64 x 576 bf16, 72 KB) goes from HBM straight into LDS (global_load_lds_dwordx4,
//     two stages); the next tile's loads are issued between the MFMAs of this tile's scores;
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 over 36 k-steps: A = K from LDS, B = the wave's
//     32 query rows kept in registers (144 VGPRs);
//   * tile row max, skip vote (ballot, LDS, barrier) exactly as in prefill;
//   * kept tiles: P = exp2(S - m) and the wave's half of O^T (256 x 32) += V^T P^T, V^T read from
//     the same LDS tile with ds_read_b64_tr_b16.
// LDS layout: a 576-wide row is 1152 bytes, so every row starts on bank 0 or 32; the 16-byte
// chunks of a row are XOR-swizzled within groups of 16 (the last 8 chunks within a group of 8)
// by the row index, which makes the 64-lane K reads conflict-free. The loads are laid out as the
// tile's bytes in order (64 chunks per wave-wide load), so each load is 1 KB of contiguous K.
// Splits write normalised partial O and base-2 LSE to the workspace; the split merge combines.
#include "internal.h"
#include "lds_dma.h"

#include <math.h>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kRowBytes = kDqk * 2;                 // 1152
constexpr int kChunks = kDqk / 8;                   // 72 chunks of 16 bytes per row
constexpr int kTileBytes = kBlockC * kRowBytes;     // 73728
constexpr int kLoadsPerTile = kTileBytes / 1024;    // 72 wave-wide 16-byte loads
constexpr int kSteps = kDqk / 16;                   // 36 k-steps of S
constexpr int kDvBlocks = kDv / 32 / 2;             // 8 output column blocks per wave

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

// Physical chunk position of logical chunk c in row r (an involution within its group).
__device__ __forceinline__ int swz(int r, int c) { return c < 64 ? (c ^ (r & 15)) : (c ^ (r & 7)); }

constexpr int NW = 4;   // waves per workgroup
constexpr int kBR = 64; // query heads per unit

template <bool PAGED>
__global__ __launch_bounds__(256, 1) void decode_mla_kernel(DecodeParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[2][kTileBytes];
  __shared__ int sVote[2][NW];
  __shared__ float sMargin[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int split = blockIdx.x;
  const int rb = blockIdx.y;
  const int b = blockIdx.z;
  const int g = 0;  // one latent KV head
  const int rg = wv & 1;   // row group of this wave
  const int half = wv >> 1; // output column half of this wave
  const int h0 = rb * kBR;
  const int my_h = h0 + rg * 32 + n;
  const bool row_ok = my_h < p.Hq && (rg * 32 + n) < p.block_r;
  int seq_len = p.kv_len ? p.kv_len[b] : p.max_kv_len;
  seq_len = max(0, min(seq_len, p.max_kv_len));
  const int seq_tiles = (seq_len + kBlockC - 1) / kBlockC;
  const int t_begin = split * p.tiles_per_split;
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
  }

  // Tile loads: wave-wide load i fills tile bytes [1024 i, 1024 i + 1024); lane L fills chunk
  // t = 64 i + L of the tile, i.e. row t / 72 at physical chunk t % 72, which holds logical
  // chunk swz(row, t % 72). This wave's load nn (0 .. 17) is wave-wide load i = wv + 4 nn.
  auto issue_one = [&](int tile, int st, int nn, int pages) {
    int ln = lane;  // opaque: recomputed per load instead of kept live across the MFMAs
    asm volatile("" : "+v"(ln));
    const int i = wv + NW * nn;
    const int t = 64 * i + ln;
    const int r = t / kChunks;
    const int pc = t - r * kChunks;
    const int key = min(tile * kBlockC + r, seq_len - 1);  // rows past the end load a real row
    int64_t roff;
    if constexpr (PAGED) {
      const int pg = __shfl(pages, key - tile * kBlockC);  // all lanes take part
      roff = (int64_t)pg * p.k_sb + (int64_t)(key & ((1 << p.page_shift) - 1)) * p.k_ss;
    } else {
      roff = (int64_t)key * p.k_ss;
    }
    const __bf16 *gp = Kg + roff + 8 * swz(r, pc);
    lds_dma16(gp, lds_addr(&smem[st][i * 1024]));
  };

  // V^T transpose-read offsets (see prefill_mfma.hip for the lane mapping): as a source lane,
  // this lane points at row 16 s + 4 (lane / 32) + (lane % 16) / 4 (+ 8) and columns
  // 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4) .. + 3 of the tile.

  f32x16_t oacc[kDvBlocks];
#pragma unroll
  for (int db = 0; db < kDvBlocks; ++db) oacc[db] = (f32x16_t)0.f;
  float m_run = -INFINITY, m_ref = -INFINITY, l_part = 0.f;
  unsigned visited = 0, skipped = 0;

  // S^T = K Q^T. K fragments are read KPF k-steps ahead of their MFMAs. The next tile's loads (next_tile >= 0) go out one per two k-steps between the MFMAs: each
  // inline-asm load is a scheduling boundary, so the reads and MFMAs between two loads stay in
  // source order, and a wave (alone on its SIMD) never stalls on a full load queue with its matrix
  // core idle.
  auto compute_s = [&](int st, f32x16_t *sacc, int next_tile, int next_pages) {
    constexpr int KPF = 2;
    sacc[0] = (f32x16_t)0.f;
    sacc[1] = (f32x16_t)0.f;
    // The per-lane offsets below do not change between tiles; the empty asm makes them opaque
    // so the compiler recomputes them (a few VALU ops) instead of keeping ~72 of them live.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int nn = ln & 31, hb = ln >> 5;
    const char *kl = smem[st] + nn * kRowBytes;
    bf16x8_t fr[kSteps][2];
    auto rd = [&](int s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int r = 32 * kb + nn;  // r & 15 == nn & 15
        fr[s][kb] = *(const bf16x8_t *)(kl + kb * 32 * kRowBytes + 16 * swz(r, 2 * s + hb));
      }
    };
#pragma unroll
    for (int s = 0; s < KPF; ++s) rd(s);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
      if (s + KPF < kSteps) rd(s + KPF);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[s][kb], qf[s], sacc[kb], 0, 0, 0);
      if ((s & 1) && next_tile >= 0) issue_one(next_tile, st ^ 1, s >> 1, next_pages);
    }
  };

  auto mask_tile = [&](int tile, f32x16_t *sacc) {
    const int k0 = tile * kBlockC;
    if (k0 + kBlockC > seq_len) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3) >= seq_len) sacc[kb][i] = -INFINITY;
    }
  };

  auto vote_tile = [&](int j, const f32x16_t *sacc) {
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = max_halves(mt);
    const float mt2 = __fmul_rn(mt, p.scale_log2);
    const float delta = (mt2 >= m_run) ? 0.f : __fsub_rn(mt2, m_run);  // exactly 0 at a new max
    m_run = fmaxf(m_run, mt2);
    const bool has_key = mt2 > -INFINITY;
    const bool keep_row = row_ok && has_key && !(delta < p.tau_log2);
    sVote[j & 1][wv] = __ballot(keep_row) != 0ull;
    if (p.tile_margin) {
      float dm = (row_ok && has_key) ? delta : -INFINITY;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) dm = fmaxf(dm, __shfl_xor(dm, o));
      sMargin[j & 1][wv] = dm;
    }
  };

  auto decision = [&](int j) {
    int keep = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) keep |= sVote[j & 1][w];  // waves of a pair vote alike
    if (tid == 0) {
      ++visited;
      skipped += keep ? 0u : 1u;
      const int64_t at = unit_tiles * p.n_tiles + t_begin + j;
      if (p.tile_status) p.tile_status[at] = keep ? 0 : 1;
      if (p.tile_margin) {
        float dm = -INFINITY;
        for (int w = 0; w < NW; ++w) dm = fmaxf(dm, sMargin[j & 1][w]);
        p.tile_margin[at] = dm * kLn2;
      }
    }
    return keep;
  };

  auto rescale_to = [&](float m_tile) {
    if (__ballot(m_tile > m_ref) != 0ull) {
      const float alpha = exp2_fast(m_ref - ((m_tile == -INFINITY) ? 0.f : m_tile));
      l_part *= alpha;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) oacc[db] *= alpha;
    }
    m_ref = m_tile;
  };

  // P = exp2(S - m) and O^T += V^T P^T, one k-step (16 keys) at a time: the 8 exponentials of a
  // step are formed right before its 16 MFMAs, so only one step's P is live.
  auto exp_pv = [&](const f32x16_t *sacc, float m_tile, int st) {
    const float m_use = (m_tile == -INFINITY) ? 0.f : m_tile;
    int ln = lane;  // opaque, as in compute_s
    asm volatile("" : "+v"(ln));
    const int vrow = 4 * (ln >> 5) + ((ln & 15) >> 2);
    const int vcb = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
    const char *vl = smem[st] + 8 * (ln & 1);
    float psum = 0.f;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = exp2_fast(fmaf(sacc[s >> 1][8 * (s & 1) + e], p.scale_log2, -m_use));
        psum += pv;
        pf[e] = (__bf16)pv;
      }
      const int r0 = 16 * s + vrow;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) {
        const int c = 4 * (kDvBlocks * half + db) + vcb;  // logical chunk (< 64)
        const char *p0 = vl + r0 * kRowBytes + 16 * (c ^ (r0 & 15));
        const char *p1 = vl + (r0 + 8) * kRowBytes + 16 * (c ^ ((r0 + 8) & 15));
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p0);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t *)p1);
        const bf16x8_t a = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, oacc[db], 0, 0, 0);
      }
    }
    l_part += psum;
  };

  // Two barriers per tile: the first publishes tile j (and frees the other stage for tile
  // j + 1, which then streams in during this tile's work), the second publishes the votes.
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
    f32x16_t sacc[2];
    compute_s(j & 1, sacc, j + 1 < n_tiles ? t_begin + j + 1 : -1, pages_next);
    mask_tile(t_begin + j, sacc);
    vote_tile(j, sacc);
    __syncthreads();
    if (decision(j)) {
      rescale_to(m_run);
      exp_pv(sacc, m_run, j & 1);
    }
  }

  // Epilogue: normalised O (or the split's partial) and LSE.
  const float l_tot = sum_halves(l_part);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (p.num_splits == 1) {
      __bf16 *orow = (__bf16 *)p.o + b * p.o_sb + (int64_t)my_h * p.o_sh + 256 * half;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = db * 32 + 8 * ig + 4 * hh;
          typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
          bf16x4_t ov = {(__bf16)(oacc[db][4 * ig + 0] * inv), (__bf16)(oacc[db][4 * ig + 1] * inv),
                         (__bf16)(oacc[db][4 * ig + 2] * inv), (__bf16)(oacc[db][4 * ig + 3] * inv)};
          *(bf16x4_t *)(orow + d0) = ov;
        }
      }
      if (p.lse && hh == 0 && half == 0)
        p.lse[(int64_t)b * p.Hq + my_h] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : -INFINITY;
    } else {
      const int64_t row = ((int64_t)b * p.Hq + my_h) * p.num_splits + split;
      float *op = p.o_part + row * kDv + 256 * half;
#pragma unroll
      for (int db = 0; db < kDvBlocks; ++db) {
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const int d0 = db * 32 + 8 * ig + 4 * hh;
          *(float4 *)(op + d0) = make_float4(oacc[db][4 * ig + 0] * inv, oacc[db][4 * ig + 1] * inv,
                                             oacc[db][4 * ig + 2] * inv, oacc[db][4 * ig + 3] * inv);
        }
      }
      if (hh == 0 && half == 0) p.lse_part[row] = l_tot > 0.f ? m_ref + __log2f(l_tot) : -INFINITY;
    }
  }
  if (tid == 0) {
    if (p.counters && visited) {
      atomicAdd(&p.counters[0], (unsigned long long)visited);
      atomicAdd(&p.counters[1], (unsigned long long)skipped);
    }
    if (p.tile_status || p.tile_margin) {
      for (int t = t_begin + n_tiles; t < t_split_end; ++t) {
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

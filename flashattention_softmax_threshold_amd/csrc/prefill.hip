// prefill.hip -- BLASST skip-softmax prefill kernel for gfx950 (CDNA4).
//
// Method: "Skip-Softmax" (vLLM-Omni design page), "Algorithm" -- FlashAttention's streaming pass
// with one test per tile: after the tile's scores are computed, the tile's softmax and P.V are
// skipped when tile_max - running_max < ln(lambda) for every query row of the tile. The pass
// itself follows "The Hitchhiker's Guide -- Phase 08", Section 1 (online softmax and the B_r x
// B_c tiling, keys in ascending order). The BLASST talk notes ("kernel design: prefill") keep
// loading V unconditionally in prefill and skip only the softmax and the second matmul; this
// kernel does the same: the V tile is staged with the K tile, and only the exp / rescale / PV
// MFMA work depends on the test.
//
// Work unit: one workgroup per (query block of B_r rows, query head, batch); NW waves of 32 rows.
// Layout on chip (one wave, lane l, row n = l % 32, half h = l / 32):
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (fp32: 32x32x2): A = K tile from LDS, B = the
//   wave's Q rows kept in registers; lane l then holds 32 scores of query row n, so the row max,
//   the running max m and the partial sum l are per-lane scalars (one swap with lane l ^ 32
//   completes a row).
//   O^T = V^T P^T: A = V^T from LDS (bf16: V is stored transposed in LDS while staging; fp32: the
//   k-width of one lets the plain row-major V serve), B = P straight from the S accumulators
//   converted to bf16. The key order inside a k-step is the accumulator's order, so P never
//   moves between lanes, and O^T's rows again belong to lane n: the rescale by alpha is a per-lane
//   multiply.
// Skip vote: per row keep = row valid && row has a visible key && !(delta < tau); a wave votes
// with a ballot, the NW waves meet through one LDS word each and a barrier; the branch is
// uniform over the workgroup.
#include "internal.h"

#include <math.h>

#include <type_traits>

namespace blasst {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

template <bool BF16, int D, int NW>
struct PrefillTraits {
  using T = typename std::conditional<BF16, __bf16, float>::type;
  static constexpr int BR = 32 * NW;   // query rows per workgroup (B_r)
  static constexpr int NT = 64 * NW;   // threads
  static constexpr int EPC = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;               // chunks per key row
  // LDS: K row-major [B_c][KP]; V: bf16 transposed [D][VP] (keys along a row), fp32 row-major.
  static constexpr int KP = D + EPC;                 // one chunk of padding per row
  static constexpr int V_ROWS = BF16 ? D : kBlockC;
  static constexpr int VP = BF16 ? kBlockC + 4 : D + EPC;
  static constexpr int K_ELEMS = kBlockC * KP;
  static constexpr int V_ELEMS = V_ROWS * VP;
  static constexpr int K_UNITS = kBlockC * CPR;                      // 16-byte chunks of K
  static constexpr int K_PER_T = (K_UNITS + NT - 1) / NT;
  static constexpr int V_UNITS = BF16 ? (kBlockC / 4) * CPR : kBlockC * CPR;  // bf16: 4 keys x 1 chunk
  static constexpr int V_PER_T = (V_UNITS + NT - 1) / NT;
  static constexpr int V_LOADS = BF16 ? 4 : 1;
};

template <bool BF16, int D, int NW>
__global__ __launch_bounds__(64 * NW) void prefill_kernel(PrefillParams p) {
  using Tr = PrefillTraits<BF16, D, NW>;
  using T = typename Tr::T;
  constexpr int BR = Tr::BR, NT = Tr::NT, EPC = Tr::EPC, CPR = Tr::CPR;
  constexpr int KP = Tr::KP, VP = Tr::VP;

  __shared__ __attribute__((aligned(16))) T sK[2][Tr::K_ELEMS];
  __shared__ __attribute__((aligned(16))) T sV[2][Tr::V_ELEMS];
  __shared__ int sVote[NW];
  __shared__ float sMargin[NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  // Causal blocks are issued longest-first (the last query block visits the most tiles).
  const int qb = p.causal ? (p.n_qblocks - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int g = hq / (p.Hq / p.Hkv);
  const T *__restrict__ Qg = (const T *)p.q + b * p.q_sb + hq * p.q_sh;
  const T *__restrict__ Kg = (const T *)p.k + b * p.k_sb + g * p.k_sh;
  const T *__restrict__ Vg = (const T *)p.v + b * p.v_sb + g * p.v_sh;
  const int blk_row0 = qb * BR;
  const int my_row = blk_row0 + wv * 32 + n;
  const bool row_ok = my_row < p.Lq;

  int n_tiles = p.n_kvtiles;
  if (p.causal) n_tiles = (min(blk_row0 + BR, p.Lq) - 1) / kBlockC + 1;
  // Sliding window: tiles before the first row's window are not visited.
  const int j0 = p.window > 0 ? max(0, blk_row0 - p.window + 1) / kBlockC : 0;

  // ---- Q fragments (B operand of S^T = K Q^T), kept in registers for the whole pass.
  constexpr int QF = BF16 ? D / 16 : D / 2;
  using QFrag = typename std::conditional<BF16, bf16x8_t, float>::type;
  QFrag qf[QF];
  {
    const T *qrow = Qg + (int64_t)(row_ok ? my_row : 0) * p.q_ss;
#pragma unroll
    for (int s = 0; s < QF; ++s) {
      if constexpr (BF16) {
        qf[s] = row_ok ? *(const bf16x8_t *)(qrow + 16 * s + 8 * hh) : (bf16x8_t)(__bf16)0.f;
      } else {
        qf[s] = row_ok ? qrow[2 * s + hh] : 0.f;
      }
    }
  }

  // ---- Tile staging: global -> registers (issued early) -> LDS (after the tile's use).
  uint4 kst[Tr::K_PER_T];
  uint4 vst[Tr::V_PER_T * Tr::V_LOADS];
  const uint4 zero4 = make_uint4(0u, 0u, 0u, 0u);

  auto load_tile = [&](int j) {
    const int k0 = j * kBlockC;
#pragma unroll
    for (int u = 0; u < Tr::K_PER_T; ++u) {
      const int idx = tid + u * NT;
      if (Tr::K_UNITS % NT == 0 || idx < Tr::K_UNITS) {
        const int key = k0 + idx / CPR, c = idx % CPR;
        kst[u] = key < p.Lkv ? *(const uint4 *)(Kg + (int64_t)key * p.k_ss + c * EPC) : zero4;
      }
    }
#pragma unroll
    for (int u = 0; u < Tr::V_PER_T; ++u) {
      const int idx = tid + u * NT;
      if (Tr::V_UNITS % NT == 0 || idx < Tr::V_UNITS) {
        if constexpr (BF16) {
          const int c = idx % CPR, kq = idx / CPR;
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int key = k0 + 4 * kq + a;
            vst[u * 4 + a] =
                key < p.Lkv ? *(const uint4 *)(Vg + (int64_t)key * p.v_ss + c * EPC) : zero4;
          }
        } else {
          const int key = k0 + idx / CPR, c = idx % CPR;
          vst[u] = key < p.Lkv ? *(const uint4 *)(Vg + (int64_t)key * p.v_ss + c * EPC) : zero4;
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < Tr::K_PER_T; ++u) {
      const int idx = tid + u * NT;
      if (Tr::K_UNITS % NT == 0 || idx < Tr::K_UNITS) {
        const int key = idx / CPR, c = idx % CPR;
        *(uint4 *)(&sK[buf][key * KP + c * EPC]) = kst[u];
      }
    }
#pragma unroll
    for (int u = 0; u < Tr::V_PER_T; ++u) {
      const int idx = tid + u * NT;
      if (Tr::V_UNITS % NT == 0 || idx < Tr::V_UNITS) {
        if constexpr (BF16) {
          // Transpose 4 keys x 8 columns: column (8c + e) of the 4 keys becomes 8 bytes of row
          // (8c + e) of V^T.
          const int c = idx % CPR, kq = idx / CPR;
          const uint32_t *x0 = (const uint32_t *)&vst[u * 4 + 0];
          const uint32_t *x1 = (const uint32_t *)&vst[u * 4 + 1];
          const uint32_t *x2 = (const uint32_t *)&vst[u * 4 + 2];
          const uint32_t *x3 = (const uint32_t *)&vst[u * 4 + 3];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int wd = e >> 1;
            uint32_t p01, p23;
            if (e & 1) {
              p01 = (x0[wd] >> 16) | (x1[wd] & 0xffff0000u);
              p23 = (x2[wd] >> 16) | (x3[wd] & 0xffff0000u);
            } else {
              p01 = (x0[wd] & 0xffffu) | (x1[wd] << 16);
              p23 = (x2[wd] & 0xffffu) | (x3[wd] << 16);
            }
            *(uint2 *)(&sV[buf][(c * 8 + e) * VP + 4 * kq]) = make_uint2(p01, p23);
          }
        } else {
          const int key = idx / CPR, c = idx % CPR;
          *(uint4 *)(&sV[buf][key * VP + c * EPC]) = vst[u];
        }
      }
    }
  };

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16_t)0.f;
  float m_run = -INFINITY;  // running row max, base-2 units
  float l_part = 0.f;       // this lane's share of the running row sum
  unsigned visited = 0, skipped = 0;
  const int64_t unit_tiles =
      (((int64_t)b * p.Hq + hq) * p.n_qblocks + qb) * (int64_t)p.n_kvtiles;

  load_tile(j0);
  store_tile(j0 & 1);
  __syncthreads();

  for (int j = j0; j < n_tiles; ++j) {
    const int buf = j & 1;
    const int k0 = j * kBlockC;
    if (j + 1 < n_tiles) load_tile(j + 1);

    // ---- S^T = K Q^T (always computed: the test needs the scores).
    f32x16_t sacc[2];
    sacc[0] = (f32x16_t)0.f;
    sacc[1] = (f32x16_t)0.f;
    const T *kl = sK[buf];
    if constexpr (BF16) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8_t a = *(const bf16x8_t *)(kl + (kb * 32 + n) * KP + 16 * s + 8 * hh);
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 2; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const float a = kl[(kb * 32 + n) * KP + 2 * s + hh];
          sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[s], sacc[kb], 0, 0, 0);
        }
      }
    }

    // ---- Mask: keys past the end, (causal) keys after the row's position and (window) keys
    // before the row's window.
    const bool need_mask = (k0 + kBlockC > p.Lkv) || (p.causal && k0 + kBlockC - 1 > blk_row0) ||
                           (p.window > 0 && k0 <= blk_row0 + BR - 1 - p.window);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = k0 + kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
          if (key >= p.Lkv || (p.causal && key > my_row) ||
              (p.window > 0 && key <= my_row - p.window))
            sacc[kb][i] = -INFINITY;
        }
      }
    }

    // ---- Tile row max, running max, and the skip vote.
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mt = fmaxf(mt, sacc[kb][i]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));
    // The row's margin tile_max - running_max (<= 0). mt2 is rounded on its own (no fused
    // multiply-add with the subtraction), and a tile holding a new row maximum gets exactly 0:
    // otherwise a contracted product could leave the new maximum a hair below 0, the row would
    // vote "skip" at lambda = 1, and the skipped tile would hold a running maximum it never set.
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
    int keep = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) keep |= sVote[w];
    if (tid == 0) {
      ++visited;
      skipped += keep ? 0u : 1u;
      if (p.tile_status) p.tile_status[unit_tiles + j] = keep ? 0 : 1;
      if (p.tile_margin) {
        float dm = -INFINITY;
        for (int w = 0; w < NW; ++w) dm = fmaxf(dm, sMargin[w]);
        p.tile_margin[unit_tiles + j] = dm * kLn2;
      }
    }

    if (keep) {
      // ---- Online-softmax update and O += P V for a kept tile.
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float psum = 0.f;
      if constexpr (BF16) {
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
        const T *vl = sV[buf];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const T *vr = vl + (db * 32 + n) * VP + 16 * s + 4 * hh;
            const bf16x4_t lo = *(const bf16x4_t *)vr;
            const bf16x4_t hi = *(const bf16x4_t *)(vr + 8);
            const bf16x8_t a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], oacc[db], 0, 0, 0);
          }
        }
      } else {
        float pv[2][16];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            pv[kb][i] = exp2_fast(fmaf(sacc[kb][i], p.scale_log2, -m_use));
            psum += pv[kb][i];
          }
        }
        l_part = fmaf(l_part, alpha, psum);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m_run = m_new;
        const T *vl = sV[buf];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kb * 32 + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const float a = vl[key * VP + db * 32 + n];
              oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, pv[kb][i], oacc[db], 0, 0, 0);
            }
          }
        }
      }
    }
    // A skipped tile leaves m, l and O alone: every valid row had tile_max < running max, so
    // the running max is unchanged.

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- Epilogue: O = acc / l, LSE = m + log l (natural log on output).
  const float l_tot = l_part + __shfl_xor(l_part, 32);
  if (row_ok) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    T *orow = (T *)p.o + b * p.o_sb + (int64_t)my_row * p.o_ss + hq * p.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = db * 32 + 8 * ig + 4 * hh;
        const float o0 = oacc[db][4 * ig + 0] * inv, o1 = oacc[db][4 * ig + 1] * inv;
        const float o2 = oacc[db][4 * ig + 2] * inv, o3 = oacc[db][4 * ig + 3] * inv;
        if constexpr (BF16) {
          bf16x4_t ov = {(__bf16)o0, (__bf16)o1, (__bf16)o2, (__bf16)o3};
          *(bf16x4_t *)(orow + d0) = ov;
        } else {
          *(float4 *)(orow + d0) = make_float4(o0, o1, o2, o3);
        }
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
      for (int j = 0; j < p.n_kvtiles; ++j) {
        if (j >= j0 && j < n_tiles) continue;
        if (p.tile_status) p.tile_status[unit_tiles + j] = 2;
        if (p.tile_margin) p.tile_margin[unit_tiles + j] = -INFINITY;
      }
    }
  }
}

template <bool BF16, int D>
hipError_t launch_d(const PrefillParams &p, int block_r, hipStream_t stream) {
  const dim3 grid(p.n_qblocks, p.Hq, p.B);
  switch (block_r) {
    case 32:
      hipLaunchKernelGGL((prefill_kernel<BF16, D, 1>), grid, dim3(64), 0, stream, p);
      break;
    case 64:
      hipLaunchKernelGGL((prefill_kernel<BF16, D, 2>), grid, dim3(128), 0, stream, p);
      break;
    case 128:
      hipLaunchKernelGGL((prefill_kernel<BF16, D, 4>), grid, dim3(256), 0, stream, p);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams &p, int dtype, int head_dim, int block_r,
                          hipStream_t stream) {
  if (dtype == 1) {
    // The MFMA kernel keeps a lane's in-tile byte offset (up to 64 rows of a stride) in 32 bits.
    const int64_t max_ss = p.k_ss > p.v_ss ? p.k_ss : p.v_ss;
    if (block_r == 128 && max_ss * 2 * kBlockC + 2 * head_dim < (int64_t(1) << 32))
      return launch_prefill_mfma(p, head_dim, stream);
    if (head_dim == 64) return launch_d<true, 64>(p, block_r, stream);
    if (head_dim == 128) return launch_d<true, 128>(p, block_r, stream);
  } else {
    if (head_dim == 64) return launch_d<false, 64>(p, block_r, stream);
    if (head_dim == 128) return launch_d<false, 128>(p, block_r, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace blasst

// MFMA GEMM engine for gfx950 shared by every expert and router GEMM of the layer.
//
// C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulation in MFMA accumulators.
//   * workgroup = 256 threads = 4 waves in a 2 x 2 grid; tile 128 (M) x 128 (N);
//   * each wave owns a 64 x 64 sub-tile = 2 x 2 MFMA 32x32 blocks
//     (bf16: v_mfma_f32_32x32x16_bf16, fp32: v_mfma_f32_32x32x2_f32);
//   * K advances in stages of 128 bytes per row (64 bf16 / 32 fp32 elements), double-buffered
//     in LDS: the next stage's global loads are in flight while the current stage feeds MFMA;
//   * both operands are staged in LDS as [row][k] (K contiguous, rows padded to 144 bytes so
//     the 32 rows one MFMA operand read touches fall on distinct banks).
//
// Operand staging (the "gather fused into the load" of the SonicMoE page, section
// "Gather 与加载融合", done with plain vector loads into LDS on gfx950):
//   * RowLoader: tile row i is a global row whose K elements are contiguous.  Its pointer comes
//     from a functor, so a row can be gathered through an index (token id of a permuted row).
//   * ColLoader: the global operand is MN-contiguous (its rows are indexed by k, possibly
//     gathered).  Each thread loads a 4 (k) x 8 (mn) block with 16-byte loads and transposes it
//     in registers before writing K-contiguous rows to LDS.
//
// Accumulator layout (32x32 MFMA, verified on gfx950): register v of lane l holds
//   row    (v / 4) * 8 + (l / 32) * 4 + (v % 4)
//   column l % 32.
#pragma once

#include "common.h"

namespace moe {

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KB = 128;                     // bytes of K per stage and row
constexpr int LDS_ROW = KB + 16;            // padded LDS row pitch (bytes)
constexpr int TILE_BYTES = 128 * LDS_ROW;   // one operand, one stage
constexpr int GEMM_LDS = 4 * TILE_BYTES;    // A and B, two stages each
constexpr int GEMM_THREADS = 256;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int BK = KB / 2;              // 64 elements per stage
  static constexpr int STEPS = BK / 16;          // MFMA k-steps per stage
  typedef bf16x8 frag;
  __device__ static frag load(const char* p) { return *reinterpret_cast<const bf16x8*>(p); }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static int off(int s, int lane) { return s * 32 + (lane >> 5) * 16; }
};
template <> struct Mma<float> {
  static constexpr int BK = KB / 4;              // 32 elements per stage
  static constexpr int STEPS = BK / 2;
  typedef float frag;
  __device__ static frag load(const char* p) { return *reinterpret_cast<const float*>(p); }
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static int off(int s, int lane) { return s * 8 + (lane >> 5) * 4; }
};

// ---------------------------------------------------------------------------------------------
// Row loader: LDS row i <- global row rp_i (K contiguous).  Thread owns rows (tid/8) + 32 q,
// 16-byte chunk (tid % 8) of each stage.  A null row pointer stages zeros.
// ---------------------------------------------------------------------------------------------
struct RowLoader {
  const char* rp[4];
  u32x4 v[4];
  int chunk;
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
    chunk = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) rp[q] = row_ptr((threadIdx.x >> 3) + 32 * q);
  }
  __device__ void load(int kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (rp[q]) v[q] = ld16(rp[q] + (int64_t)kt * KB + chunk * 16);
      else v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(lds + ((threadIdx.x >> 3) + 32 * q) * LDS_ROW + chunk * 16) = v[q];
  }
};

// ---------------------------------------------------------------------------------------------
// Column loader: the operand element (mn, k) lives at kptr(k) + mn * sizeof(T) (global rows are
// indexed by k).  Thread loads rows k0..k0+3 of one 16-byte mn chunk and writes the transposed
// block as K-contiguous LDS rows.  kptr returns null for k outside the operand (zeros), and mn
// chunks at or beyond mn_valid are zero.
// ---------------------------------------------------------------------------------------------
template <typename T>
struct ColLoader {
  static constexpr int VEC = 16 / sizeof(T);           // mn elements per chunk (8 or 4)
  static constexpr int MNB = 128 / VEC;                // chunks across the tile (16 or 32)
  u32x4 v[4];
  int mnb, kq;
  bool mn_ok;
  __device__ void init(int mn_base, int mn_valid) {
    mnb = threadIdx.x % MNB;
    kq = threadIdx.x / MNB;
    mn_ok = mn_base + mnb * VEC < mn_valid;
  }
  // kptr(k) -> const char* (already including the mn_base offset) or nullptr.
  template <class KPtr>
  __device__ void load(int kt, KPtr kptr) {
    const int k0 = kt * Mma<T>::BK + kq * 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const char* p = mn_ok ? kptr(k0 + kk) : nullptr;
      if (p) v[kk] = ld16(p + mnb * 16);
      else v[kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = 16 * (e & 1), w = e >> 1;
        u32x2 o;
        o[0] = ((v[0][w] >> sh) & 0xffffu) | (((v[1][w] >> sh) & 0xffffu) << 16);
        o[1] = ((v[2][w] >> sh) & 0xffffu) | (((v[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(lds + (mnb * 8 + e) * LDS_ROW + kq * 8) = o;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 o{v[0][e], v[1][e], v[2][e], v[3][e]};
        *reinterpret_cast<u32x4*>(lds + (mnb * 4 + e) * LDS_ROW + kq * 16) = o;
      }
    }
  }
};

// One stage of MFMA work for this wave.  bsub(j) = first LDS row of the wave's j-th B block.
template <typename T, class BSub>
__device__ __forceinline__ void mma_stage(const char* As, const char* Bs, f32x16 (&acc)[2][2],
                                          int wm, BSub bsub) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int s = 0; s < Mma<T>::STEPS; ++s) {
    typename Mma<T>::frag a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = Mma<T>::load(As + (wm * 64 + i * 32 + (lane & 31)) * LDS_ROW + Mma<T>::off(s, lane));
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = Mma<T>::load(Bs + (bsub(j) + (lane & 31)) * LDS_ROW + Mma<T>::off(s, lane));
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = Mma<T>::mma(a[i], b[j], acc[i][j]);
  }
}

// Double-buffered main loop over `nkt` K stages.  `la` / `lb` expose load(kt) and store(lds).
template <typename T, class LA, class LB, class BSub>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nkt, f32x16 (&acc)[2][2],
                                              char* lds, int wm, BSub bsub) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  if (nkt <= 0) return;
  char* As0 = lds;
  char* Bs0 = lds + TILE_BYTES;
  char* As1 = lds + 2 * TILE_BYTES;
  char* Bs1 = lds + 3 * TILE_BYTES;
  la.load(0);
  lb.load(0);
  la.store(As0);
  lb.store(Bs0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool odd = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
    mma_stage<T>(odd ? As1 : As0, odd ? Bs1 : Bs0, acc, wm, bsub);
    if (more) {
      la.store(odd ? As0 : As1);
      lb.store(odd ? Bs0 : Bs1);
    }
    __syncthreads();
  }
}

// Row (within the 128-row tile) of accumulator register v for this lane and M block i.
__device__ __forceinline__ int acc_row(int wm, int i, int v) {
  const int lane = threadIdx.x & 63;
  return wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}

// Grouped M tiles: tile mt of the concatenation of experts' ceil(rows/128) tiles.
struct GroupTile {
  int e, m0, mrows;
};
__device__ __forceinline__ bool find_group_tile(int mt, const int32_t* __restrict__ mtile_off,
                                                const int32_t* __restrict__ expert_off, int E,
                                                GroupTile& g) {
  if (mt >= mtile_off[E]) return false;
  int lo = 0, hi = E;  // mtile_off[lo] <= mt < mtile_off[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mtile_off[mid] <= mt) lo = mid;
    else hi = mid;
  }
  g.e = lo;
  g.m0 = expert_off[lo] + (mt - mtile_off[lo]) * BM;
  g.mrows = min(BM, expert_off[lo + 1] - g.m0);
  return true;
}

}  // namespace moe

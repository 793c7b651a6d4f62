// MFMA GEMM engine for gfx950, shared by every expert and router GEMM of the layer.
//
// C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulation in MFMA accumulators.
//   * workgroup = 512 threads = 8 waves in a 2 (M) x 4 (N) grid; block tile 256 x 256;
//   * each wave owns 128 x 64 = 4 x 2 MFMA 32x32 blocks
//     (bf16: v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2_f32);
//   * K advances in stages of 128 bytes per row (64 bf16 / 32 fp32 elements), double-buffered in
//     LDS: the next stage's global loads are in flight while the current stage feeds the MFMAs.
//
// Operand staging (the SonicMoE page's "gather fused into the HBM->SMEM load", done on gfx950 with
// 16-byte vector loads into LDS; a row pointer can come through an index, so gathered token rows
// cost nothing extra):
//   * K-major operand (each row's K elements contiguous in memory, e.g. activations or
//     [out][in] weights): LDS tile [256 rows][128 B + 16 B pad]; an MFMA fragment is one
//     ds_read_b128 (32 lanes on 32 rows: the 144-byte pitch puts them on distinct banks).
//   * MN-major bf16 operand (each k-row contiguous along M or N, e.g. dY / X / dH rows feeding a
//     weight gradient, or weights read transposed): staged untransposed as LDS [64 k][256 mn]
//     with a 576-byte pitch, and read with the gfx950 transposing LDS load ds_read_b64_tr_b16.
//     Within a 16-lane group, lane i supplies 4 consecutive 16-bit elements and lane j receives
//     element j%4 of lanes j/4, j/4+4, j/4+8, j/4+12 (verified on gfx950).  Lane i therefore
//     points at k-row i/4 and column 4(i%4): lane j receives 4 consecutive k of column j.  Two
//     such loads give the 8 k-values of an MFMA fragment.  The 576-byte pitch (= 16 banks mod 64)
//     puts the four k-rows one half-wave touches on disjoint banks.
//   * MN-major fp32 operands (small fp32 layers only) are transposed in registers while staged.
//
// Accumulator layout (32x32 MFMA, verified on gfx950): register v of lane l holds
//   row (v / 4) * 8 + (l / 32) * 4 + (v % 4), column l % 32.
#pragma once

#include "common.h"

namespace moe {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int GEMM_THREADS = 512;
constexpr int KB = 128;                     // bytes of K per stage and row
constexpr int KROW = KB + 16;               // K-major LDS row pitch
constexpr int MNROW = 256 * 2 + 64;         // MN-major (bf16) LDS row pitch
constexpr int STAGE_BYTES = 256 * KROW;     // one operand, one stage (= 64 * MNROW)
static_assert(STAGE_BYTES == 64 * MNROW, "operand stage sizes must agree");
constexpr int GEMM_LDS = 4 * STAGE_BYTES;   // A and B, two stages each: 147456 bytes

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int BK = KB / 2;              // 64 elements per stage
  static constexpr int STEPS = BK / 16;
  typedef bf16x8 frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int BK = KB / 4;              // 32 elements per stage
  static constexpr int STEPS = BK / 2;
  typedef float frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------------------------
// Fragment readers.  row0 / mn0: first of the 32 rows (M or N) of the fragment; s: k-step.
// ---------------------------------------------------------------------------------------------
template <typename T> struct KFrag;
template <> struct KFrag<bf16> {
  __device__ static bf16x8 read(const char* lds, int row0, int s) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const bf16x8*>(lds + (row0 + (lane & 31)) * KROW + s * 32 + (lane >> 5) * 16);
  }
};
template <> struct KFrag<float> {
  __device__ static float read(const char* lds, int row0, int s) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const float*>(lds + (row0 + (lane & 31)) * KROW + s * 8 + (lane >> 5) * 4);
  }
};
struct MNFrag {  // bf16 only
  __device__ static bf16x8 read(const char* lds, int mn0, int s) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i = lane & 15;
    const int k = s * 16 + (g >> 1) * 8 + (i >> 2);
    const int mn = mn0 + (g & 1) * 16 + 4 * (i & 3);
    const char* p = lds + k * MNROW + mn * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * MNROW));
    const v4i16 both[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, both, 16);
    return r;
  }
};

// ---------------------------------------------------------------------------------------------
// Loaders: load(kt) issues the global loads of stage kt into registers, store(lds) writes them.
// ---------------------------------------------------------------------------------------------
// K-major rows: LDS row i <- 128 bytes of global row rp_i at stage kt.  Thread owns rows
// tid/8 + 64 q (q = 0..3), chunk tid % 8.  A null row stages zeros.
struct RowLoader {
  const char* rp[4];
  u32x4 v[4];
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
#pragma unroll
    for (int q = 0; q < 4; ++q) rp[q] = row_ptr((threadIdx.x >> 3) + 64 * q);
  }
  __device__ void load(int kt) {
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (rp[q]) v[q] = ld16(rp[q] + (int64_t)kt * KB + chunk * 16);
      else v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(lds + ((threadIdx.x >> 3) + 64 * q) * KROW + chunk * 16) = v[q];
  }
};

// MN-major bf16 tile, staged untransposed: LDS [64 k][256 mn].  kptr(k) returns the global
// address of element (mn_base, k) or null (zeros).  Thread owns k-rows tid/32 + 16 q, chunk
// tid % 32 (8 mn elements); chunks at or beyond mn_valid stage zeros.
template <class KPtr>
struct TileLoaderMN {
  KPtr kptr;
  u32x4 v[4];
  bool ok;
  __device__ TileLoaderMN(KPtr f, int mn_base, int mn_valid) : kptr(f) {
    ok = mn_base + (int)(threadIdx.x & 31) * 8 < mn_valid;
  }
  __device__ void load(int kt) {
    const int chunk = threadIdx.x & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const char* p = ok ? kptr(kt * 64 + (int)(threadIdx.x >> 5) + 16 * q) : nullptr;
      if (p) v[q] = ld16(p + chunk * 16);
      else v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
    const int chunk = threadIdx.x & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<u32x4*>(lds + ((threadIdx.x >> 5) + 16 * q) * MNROW + chunk * 16) = v[q];
  }
};

// MN-major fp32 operand, transposed in registers into the K-major LDS layout: thread owns a
// 4 (k) x 4 (mn) block, mn = 4 (tid % 64), k = 4 (tid / 64).
template <class KPtr>
struct ColLoaderF32 {
  KPtr kptr;
  u32x4 v[4];
  bool ok;
  __device__ ColLoaderF32(KPtr f, int mn_base, int mn_valid) : kptr(f) {
    ok = mn_base + (int)(threadIdx.x & 63) * 4 < mn_valid;
  }
  __device__ void load(int kt) {
    const int k0 = kt * Mma<float>::BK + (int)(threadIdx.x >> 6) * 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const char* p = ok ? kptr(k0 + kk) : nullptr;
      if (p) v[kk] = ld16(p + (threadIdx.x & 63) * 16);
      else v[kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
    const int mn0 = (threadIdx.x & 63) * 4, kq = threadIdx.x >> 6;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      u32x4 o{v[0][e], v[1][e], v[2][e], v[3][e]};
      *reinterpret_cast<u32x4*>(lds + (mn0 + e) * KROW + kq * 16) = o;
    }
  }
};

// The MN-major operand kind for element type T: loader type and fragment reader.
template <typename T, class KPtr> struct MNOperand;
template <class KPtr> struct MNOperand<bf16, KPtr> {
  typedef TileLoaderMN<KPtr> Loader;
  __device__ static bf16x8 frag(const char* lds, int mn0, int s) { return MNFrag::read(lds, mn0, s); }
};
template <class KPtr> struct MNOperand<float, KPtr> {
  typedef ColLoaderF32<KPtr> Loader;
  __device__ static float frag(const char* lds, int mn0, int s) { return KFrag<float>::read(lds, mn0, s); }
};
template <typename T> struct KOperand {
  typedef RowLoader Loader;
  __device__ static typename Mma<T>::frag frag(const char* lds, int row0, int s) {
    return KFrag<T>::read(lds, row0, s);
  }
};

// ---------------------------------------------------------------------------------------------
// Main loop.  AOp / BOp provide frag(lds, first_row, kstep); la / lb the loaders.  bsub(j) is the
// first LDS row (N index) of the wave's j-th B block.  Accumulators acc[i][j]: M block i of the
// wave's 128 rows, N block j of its two 32-column blocks.
// ---------------------------------------------------------------------------------------------
struct WaveAcc {
  f32x16 c[4][2];
};

template <typename T, class AOp, class BOp, class LA, class LB, class BSub>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nkt, WaveAcc& acc, char* lds,
                                              int wm, BSub bsub) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nkt <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(lds);
  lb.store(lds + STAGE_BYTES);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const char* As = lds + (kt & 1) * 2 * STAGE_BYTES;
    const char* Bs = As + STAGE_BYTES;
    const bool more = kt + 1 < nkt;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
#pragma unroll
    for (int s = 0; s < Mma<T>::STEPS; ++s) {
      typename Mma<T>::frag a[4], b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = BOp::frag(Bs, bsub(j), s);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = AOp::frag(As, wm * 128 + i * 32, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc.c[i][j] = Mma<T>::mma(a[i], b[j], acc.c[i][j]);
    }
    if (more) {
      char* Ad = lds + ((kt + 1) & 1) * 2 * STAGE_BYTES;
      la.store(Ad);
      lb.store(Ad + STAGE_BYTES);
    }
    __syncthreads();
  }
}

// Tile row of accumulator register v for M block i of wave row wm.
__device__ __forceinline__ int acc_row(int wm, int i, int v) {
  const int lane = threadIdx.x & 63;
  return wm * 128 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
}

// ---------------------------------------------------------------------------------------------
// Epilogue through LDS for 2-byte outputs: the wave writes val(i, j, v) at (acc_row, col(j)) of a
// [256][ncols] bf16 staging tile, then the block stores rows < mrows and columns < ncols_valid
// with 16-byte writes: out + r * ld (elements) + c.  Requires the LDS to be free (after the
// main loop) and ncols <= 256.
// ---------------------------------------------------------------------------------------------
constexpr int EPI_ROW = 256 * 2 + 16;

template <class Col, class Val>
__device__ __forceinline__ void epi_stage_bf16(char* lds, const WaveAcc& acc, int wm, Col col, Val val) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = col(j);
    if (c < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        *reinterpret_cast<bf16*>(lds + acc_row(wm, i, v) * EPI_ROW + c * 2) = (bf16)val(i, j, v);
  }
}

__device__ __forceinline__ void epi_store_bf16(const char* lds, bf16* out, int64_t ld, int mrows,
                                               int ncols, int ncols_valid) {
  const int cpr = ncols / 8;  // 16-byte chunks per row
  for (int c = threadIdx.x; c < 256 * cpr; c += GEMM_THREADS) {
    const int r = c / cpr, ch = c % cpr;
    if (r < mrows && ch * 8 < ncols_valid)
      st16(out + (int64_t)r * ld + ch * 8, *reinterpret_cast<const u32x4*>(lds + r * EPI_ROW + ch * 16));
  }
}

// Grouped M tiles: tile mt of the concatenation of the experts' ceil(rows / BM) tiles.
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

// Backward of the MoE layer: dAct GEMM with the SwiGLU backward and router-score partials in its
// epilogue, the weight-gradient GEMMs that reduce over each expert's rows, the dX GEMM, and the
// router backward fused with the scatter-free dX gather-sum.
//
// Pages: SonicMoE page, optimization 1 (nothing the router gradient needs is cached; A is
// recomputed from the cached pre-activations), section "反向传播优化" (dW1 reads gathered X,
// dW2 and dH read gathered dO, each gather fused into the GEMM's operand load), and the
// kernel-comparison table ("dS computation": dS_r = <dY_t W_down[e], A_r>, which equals
// <dY_t, Y_r> without the expert output Y ever being stored).
#include "gemm_core.h"
#include "internal.h"

namespace moe {

static inline int grid8(int64_t n) { return (int)((n + 7) / 8 * 8); }

// ---------------------------------------------------------------------------------------------
// dAct: dA'[r][j] = sum_c dY[t_r][c] W_down[e][c][j]  (M = rows of e, N = n, K = d).
// Wave column wn owns columns (j/2)*128 + wn*64 + (j%2)*32 + (lane % 32), j = 0..3, so that
// each 128-column half of the tile holds two of its blocks and can be finished on its own.
// Epilogue per (r, j), with G, U read from H and w = row_w[r]:
//   A = silu(G) U;  dS partial += dA' A;  dA = w dA'
//   dG = dA U sigmoid(G) (1 + G (1 - sigmoid(G)));  dU = dA silu(G)
//   dH[r] = [dG | dU];  wA[r][j] = w A   (the down-weight gradient's operand)
// dS partials are reduced over the tile's columns in registers, lanes and LDS, and written per
// column tile: dS_part[nt][r].
// ---------------------------------------------------------------------------------------------
// The dAct epilogue of one tile, one 128-column half at a time: dump(half, frow) writes the
// waves' fp32 accumulators of that half into an LDS tile [256][128] (row r at frow(r)), then the
// block walks the half row by row in 16-byte chunks (coalesced loads of G, U and coalesced
// stores of dG, dU, w A), and the 16 or 32 lanes that share a row reduce its dS partial.  The
// block walks chunk c = row * CPR + ch in batches of UNR chunks per thread; the G, U and
// row-weight loads of PF batches go out together -- the first group before the accumulator dump
// and its barrier -- so a group costs one memory round trip, not one per batch.
template <typename T, int NTHR, int PF, class Dump>
__device__ __forceinline__ void dact_epilogue(LdsBufs L, const GroupTile& g, int n0, int n, int nt, int64_t R_max,
                                              const float* __restrict__ row_w, const T* __restrict__ H,
                                              T* __restrict__ dH, T* __restrict__ wA, float* __restrict__ dS_part,
                                              Dump dump) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = 128 / VEC;                 // chunks per half-row
  constexpr int FROW = 128 * 4 + 16;             // fp32 staging pitch
  static_assert(64 * FROW + 1024 <= LDS_BUF, "fp32 staging + dS partials");
  float* red = reinterpret_cast<float*>(L.b[0] + 64 * FROW);  // [256] dS partials of this tile
  auto frow = [&](int r) { return epi_buf(L, r) + (r & 63) * FROW; };
  const int valid = min(BN, n - n0);
  constexpr int UNR = 4;
  constexpr int NB = 256 * CPR / (UNR * NTHR);  // batches per half
  static_assert(NB * UNR * NTHR == 256 * CPR, "whole batches");
  static_assert(NB % PF == 0, "whole groups");
  auto chunk_at = [&](int half, int b, int u, int& row, int& ch, int& col) {
    const int c = (b * UNR + u) * NTHR + threadIdx.x;
    row = c / CPR;
    ch = c % CPR;
    col = half * 128 + ch * VEC;
    return row < g.mrows && col < valid;
  };
  // G, U and the row weight of UNR chunks; H is read once and the outputs are not read again by
  // this kernel, so both go around the caches' retention (non-temporal)
  struct Grp {
    u32x4 g[UNR], u[UNR];
    float w[UNR];
  };
  // Every thread issues the same number of loads whatever its chunks' validity (an invalid chunk
  // reads the tile's last valid row and column chunk, and its values go unused), so the waits
  // that follow can count them.
  auto load_grp = [&](int half, int b, Grp& q) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      int row, ch, col;
      chunk_at(half, b, u, row, ch, col);
      const int64_t r = g.m0 + min(row, g.mrows - 1);
      const int c = min(col, valid - VEC);
      q.g[u] = ld16_nt(H + r * 2 * n + n0 + c);
      q.u[u] = ld16_nt(H + r * 2 * n + n + n0 + c);
      q.w[u] = row_w[r];
    }
  };
  // The arithmetic runs for every chunk (an invalid one on the stand-in values above and the
  // zero rows of the staged tile), so that the loaded values are used on every path and the
  // compiler keeps the loads where they are issued; only the stores and the dS term are masked.
  auto run_grp = [&](int half, int b, const Grp& q) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      int row, ch, col;
      const bool ok = chunk_at(half, b, u, row, ch, col);
      const int64_t r = g.m0 + row;
      const float w = q.w[u];
      float p = 0.0f;
      float dAp[VEC], G[VEC], U[VEC], oG[VEC], oU[VEC], oA[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) dAp[k] = *reinterpret_cast<const float*>(frow(row) + (ch * VEC + k) * 4);
      unpack16<T>(q.g[u], G);
      unpack16<T>(q.u[u], U);
#pragma unroll
      for (int k = 0; k < VEC; ++k) {
        const float sg = sigmoid_f32(G[k]);
        const float silu = G[k] * sg;
        const float A = silu * U[k];
        p += dAp[k] * A;
        const float dA = w * dAp[k];
        oG[k] = dA * U[k] * sg * (1.0f + G[k] * (1.0f - sg));
        oU[k] = dA * silu;
        oA[k] = w * A;
      }
      if (ok) {
        st16_nt(dH + r * 2 * n + n0 + col, pack16<T>(oG));
        st16_nt(dH + r * 2 * n + n + n0 + col, pack16<T>(oU));
        st16_nt(wA + r * n + n0 + col, pack16<T>(oA));
      }
      p = ok ? p : 0.0f;
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) p += __shfl_xor(p, o, 64);
      if (ch == 0) red[row] = half == 0 ? p : red[row] + p;
    }
  };
  if constexpr (NB == 2 && PF == 2) {
    // two batches per half (eight waves): the first half's first batch goes out before its dump,
    // its second batch and the second half's first batch right after the dump, and the second
    // half's second batch once the first half is done (before its stores drain), so that the
    // second half's loads are not queued behind the first half's stores; the registers of both
    // halves' batches do not fit at once.  Scheduling barriers keep the loads in this order,
    // which the waits count on.
    Grp a0, a1, b0, b1;
    load_grp(0, 0, a0);
    __builtin_amdgcn_sched_barrier(0);
    dump(0, frow);
    __builtin_amdgcn_sched_barrier(0);
    load_grp(0, 1, a1);
    load_grp(1, 0, b0);
    __syncthreads();
    run_grp(0, 0, a0);
    run_grp(0, 1, a1);
    __builtin_amdgcn_sched_barrier(0);
    load_grp(1, 1, b1);
    __syncthreads();
    dump(1, frow);
    __syncthreads();
    run_grp(1, 0, b0);
    run_grp(1, 1, b1);
    __syncthreads();
  } else {
    Grp q[PF];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int pb = 0; pb < PF; ++pb) load_grp(half, pb, q[pb]);
      dump(half, frow);
      __syncthreads();
#pragma unroll 1
      for (int b0 = 0; b0 < NB; b0 += PF) {
        if (b0 > 0)
#pragma unroll
          for (int pb = 0; pb < PF; ++pb) load_grp(half, b0 + pb, q[pb]);
#pragma unroll
        for (int pb = 0; pb < PF; ++pb) run_grp(half, b0 + pb, q[pb]);
      }
      __syncthreads();
    }
  }
  if (threadIdx.x < 256 && (int)threadIdx.x < g.mrows)
    dS_part[(int64_t)nt * R_max + g.m0 + threadIdx.x] = red[threadIdx.x];
}

template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_dact(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const float* __restrict__ row_w,
    const T* __restrict__ dY, const T* __restrict__ Wd, const T* __restrict__ H,
    T* __restrict__ dH, T* __restrict__ wA, float* __restrict__ dS_part, int64_t R_max, int d,
    int n, int E, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int nt = g.nt;
  const int n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)d * sizeof(T);
  auto la = k_rows<T>([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(dY) + (int64_t)clamp_idx(row_token[g.m0 + i], T_) * rowb
                       : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wd) + ((int64_t)g.e * d * n + n0) * sizeof(T);
  auto lb = mn_rows<T>([=](int k) { return wd + (int64_t)k * n * sizeof(T); }, d, n0, n);
  WaveAcc acc;
  gemm_mainloop<T>(la, lb, d / Mma<T>::BK, acc, L, wm, [&](int j) { return bsub_halved(wn, j); });
  // half h holds the wave's blocks j = 2 h and 2 h + 1 (halved layout)
  dact_epilogue<T, GEMM_THREADS, sizeof(T) == 2 ? 2 : 1>(L, g, n0, n, nt, R_max, row_w, H, dH, wA, dS_part,
                                                         [&](int half, auto frow) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v4 = {acc.c[i][2 * half + jj][4 * q], acc.c[i][2 * half + jj][4 * q + 1],
                            acc.c[i][2 * half + jj][4 * q + 2], acc.c[i][2 * half + jj][4 * q + 3]};
          *reinterpret_cast<f32x4*>(frow(acc_m(wm, i)) + (wn * 64 + jj * 32 + acc_n(4 * q)) * 4) = v4;
        }
  });
}

// bf16 dAct on the eight-wave engine (same tiles, operands and bits as k_dact).  Block j of wave
// column wn covers columns j * 128 + wn * 32 .. + 31, so half h of the tile holds each wave's
// block h.
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_dact_w8(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const float* __restrict__ row_w,
    const bf16* __restrict__ dY, const bf16* __restrict__ Wd, const bf16* __restrict__ H,
    bf16* __restrict__ dH, bf16* __restrict__ wA, float* __restrict__ dS_part, int64_t R_max, int d,
    int n, int E, int NT, int T_, int light_last) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  const bool found = light_last ? find_group_tile<true>(lin, NT, mtile_off, expert_off, E, g)
                                : find_group_tile<false>(lin, NT, mtile_off, expert_off, E, g);
  if (!found) return;
  const int nt = g.nt;
  const int n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t rowb = (int64_t)d * sizeof(bf16);
  KDmaW8 la;
  la.init([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(dY) + (int64_t)clamp_idx(row_token[g.m0 + i], T_) * rowb
                       : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wd) + ((int64_t)g.e * d * n + n0) * sizeof(bf16);
  auto lb = mn_rows_w8([=](int k) { return wd + (int64_t)k * n * sizeof(bf16); }, d, n0, n);
  AccW8 acc;
  gemm_mainloop_w8_rows(la, lb, d / Mma<bf16>::BK, acc, L, wm, [&](int j) { return j * 128 + wn * 32; }, g.mrows);
  dact_epilogue<bf16, GEMM8_THREADS, 2>(L, g, n0, n, nt, R_max, row_w, H, dH, wA, dS_part, [&](int half, auto frow) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 v4 = {acc.c[i][half][4 * q], acc.c[i][half][4 * q + 1], acc.c[i][half][4 * q + 2],
                          acc.c[i][half][4 * q + 3]};
        *reinterpret_cast<f32x4*>(frow(acc_m(wm, i)) + (wn * 32 + acc_n(4 * q)) * 4) = v4;
      }
  });
}

int dact_ntiles(int64_t n) { return (int)cdiv(n, BN); }

hipError_t launch_dact_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                            const void* dY, const void* W_down, const void* H, void* dH, void* wA,
                            float* dS_part, hipStream_t st) {
  const int NT = dact_ntiles(s.n);
  const int64_t tiles = max_mtiles(s.R_max, s.E) * NT;
  const int grid = grid8(tiles);
  // Light tails last pays while the grid is a few rounds (its last partial round is then a large
  // share of the kernel); with many rounds their weight slices, read again far from the rest of
  // their expert, cost more (measured at 4 and 43 rounds of 256 workgroups).
  const int light_last = tiles <= 8 * 256 ? 1 : 0;
  if (s.bf16)
    k_dact_w8<<<grid, GEMM8_THREADS, 0, st>>>(mtile_off, p.expert_off, p.row_token, p.row_w, (const bf16*)dY,
                                              (const bf16*)W_down, (const bf16*)H, (bf16*)dH, (bf16*)wA, dS_part,
                                              s.R_max, (int)s.d, (int)s.n, s.E, NT, (int)s.T, light_last);
  else
    k_dact<float><<<grid, GEMM_THREADS, 0, st>>>(mtile_off, p.expert_off, p.row_token, p.row_w,
                                                 (const float*)dY, (const float*)W_down, (const float*)H,
                                                 (float*)dH, (float*)wA, dS_part, s.R_max, (int)s.d,
                                                 (int)s.n, s.E, NT, (int)s.T);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// dX_perm[r][c] = sum_j dG[r][j] W_gate[e][j][c] + dU[r][j] W_up[e][j][c]
// (M = rows of e, N = d, K = 2n: k < n walks W_gate, k >= n walks W_up; B is MN-major).
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_dx(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const T* __restrict__ dH, const T* __restrict__ Wg, const T* __restrict__ Wu,
    T* __restrict__ dXp, int d, int n, int E, int NT) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int nt = g.nt;
  const int n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)2 * n * sizeof(T);
  auto la = k_rows<T>([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(dH) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const int64_t wrow = (int64_t)d * sizeof(T);
  const char* wg = reinterpret_cast<const char*>(Wg) + (int64_t)g.e * n * wrow + n0 * sizeof(T);
  const char* wu = reinterpret_cast<const char*>(Wu) + (int64_t)g.e * n * wrow + n0 * sizeof(T);
  auto lb = mn_rows<T>([=](int k) { return k < n ? wg + (int64_t)k * wrow : wu + (int64_t)(k - n) * wrow; },
                       2 * n, n0, d);
  WaveAcc acc;
  gemm_mainloop<T>(la, lb, 2 * n / Mma<T>::BK, acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  const int valid = min(BN, d - n0);
  if constexpr (sizeof(T) == 2) {
    epi_stage_bf16(L, wm, [&](int j) { return bsub_plain(wn, j); },
                   [&](int i, int j, int v) { return acc.c[i][j][v]; });
    __syncthreads();
    epi_store_bf16(L, 0, reinterpret_cast<bf16*>(dXp) + (int64_t)g.m0 * d + n0, d, g.mrows, BN, valid);
  } else {
    epi_store_direct(wm, wn, acc, valid, g.mrows, [&](int m) { return dXp + (int64_t)(g.m0 + m) * d + n0; });
  }
}

// bf16 dX on the eight-wave engine (same tiles, operands and bits as k_dx).
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_dx_w8(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const bf16* __restrict__ dH, const bf16* __restrict__ Wg, const bf16* __restrict__ Wu,
    bf16* __restrict__ dXp, int d, int n, int E, int NT) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap<64>(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t rowb = (int64_t)2 * n * sizeof(bf16);
  KDmaW8 la;
  la.init([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(dH) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const int64_t wrow = (int64_t)d * sizeof(bf16);
  const char* wg = reinterpret_cast<const char*>(Wg) + (int64_t)g.e * n * wrow + n0 * sizeof(bf16);
  const char* wu = reinterpret_cast<const char*>(Wu) + (int64_t)g.e * n * wrow + n0 * sizeof(bf16);
  auto lb = mn_rows_w8([=](int k) { return k < n ? wg + (int64_t)k * wrow : wu + (int64_t)(k - n) * wrow; },
                       2 * n, n0, d);
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_w8_rows(la, lb, 2 * n / Mma<bf16>::BK, acc, L, wm, bsub, g.mrows);
  const int valid = min(BN, d - n0);
  epi_stage_w8(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v]; });
  __syncthreads();
  bf16* out = dXp + (int64_t)g.m0 * d + n0;
  epi_store_rows<GEMM8_THREADS>(L, 0, [&](int r) { return out + (int64_t)r * d; }, g.mrows, BN, valid);
}

hipError_t launch_dx_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                          const void* dH, const void* W_gate, const void* W_up, void* dX_perm,
                          hipStream_t st) {
  const int NT = (int)cdiv(s.d, BN);
  const int grid = grid8(max_mtiles(s.R_max, s.E) * NT);
  if (s.bf16)
    k_dx_w8<<<grid, GEMM8_THREADS, 0, st>>>(mtile_off, p.expert_off, (const bf16*)dH, (const bf16*)W_gate,
                                            (const bf16*)W_up, (bf16*)dX_perm, (int)s.d, (int)s.n, s.E, NT);
  else
    k_dx<float><<<grid, GEMM_THREADS, 0, st>>>(mtile_off, p.expert_off, (const float*)dH,
                                               (const float*)W_gate, (const float*)W_up, (float*)dX_perm,
                                               (int)s.d, (int)s.n, s.E, NT);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Weight gradients: one output tile of one expert per workgroup; K runs over the expert's rows.
//   dW_down[e][c][j] = sum_r dY[t_r][c] wA[r][j]          (M = d, N = n)
//   dW_gu[e][j][c]   = sum_r dH[r][j] X[t_r][c]           (M = 2n, N = d; j < n -> gate)
// Both operands are MN-major in memory (their rows are the expert's token rows); bf16 tiles are
// staged as they lie and read with the transposing LDS load.  Experts without rows get zero
// tiles.
// ---------------------------------------------------------------------------------------------
// The expert order of these GEMMs (order[rank] = e, decreasing row count, ties to the lower id) is
// computed with the tile offsets (k_tile_offsets).  The weight-gradient GEMMs reduce over an
// expert's rows, so their tiles take time in proportion to its count; taking the experts in this
// order starts the longest tiles first and leaves the short ones to fill the end of the grid,
// instead of a hot expert's tiles forming the tail.
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_dw_down(
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ order, const int32_t* __restrict__ row_token,
    const T* __restrict__ dY, const T* __restrict__ wA, T* __restrict__ dWd, int d, int n,
    int E, int MT, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  if (lin / per >= E) return;
  const int e = order[lin / per];
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int off = expert_off[e];
  const int cnt = expert_off[e + 1] - off;
  const char* dyb = reinterpret_cast<const char*>(dY) + m0 * sizeof(T);
  const char* wab = reinterpret_cast<const char*>(wA) + n0 * sizeof(T);
  auto la = mn_rows_idx<T>([=](int k) { return clamp_idx(sload_i32(row_token + off, k), T_); },
                          [=](int t) { return dyb + (int64_t)t * d * sizeof(T); }, cnt, m0, d);
  auto lb = mn_rows<T>([=](int k) { return wab + (int64_t)(off + k) * n * sizeof(T); }, cnt, n0, n);
  WaveAcc acc;
  gemm_mainloop<T>(la, lb, (int)cdiv(cnt, Mma<T>::BK), acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  T* out = dWd + (int64_t)e * d * n;
  const int mrows = min(BM, d - m0), valid = min(BN, n - n0);
  if constexpr (sizeof(T) == 2) {
    epi_stage_bf16(L, wm, [&](int j) { return bsub_plain(wn, j); },
                   [&](int i, int j, int v) { return acc.c[i][j][v]; });
    __syncthreads();
    epi_store_bf16(L, 0, reinterpret_cast<bf16*>(out) + (int64_t)m0 * n + n0, n, mrows, BN, valid);
  } else {
    epi_store_direct(wm, wn, acc, valid, mrows, [&](int m) { return out + (int64_t)(m0 + m) * n + n0; });
  }
}

// bf16 dW_down on the eight-wave engine (same tiles, operands and bits as k_dw_down).
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_dw_down_w8(
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ order, const int32_t* __restrict__ row_token,
    const bf16* __restrict__ dY, const bf16* __restrict__ wA, bf16* __restrict__ dWd, int d, int n,
    int E, int MT, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  if (lin / per >= E) return;
  const int e = order[lin / per];
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int off = expert_off[e];
  const int cnt = expert_off[e + 1] - off;
  const char* dyb = reinterpret_cast<const char*>(dY) + m0 * sizeof(bf16);
  const char* wab = reinterpret_cast<const char*>(wA) + n0 * sizeof(bf16);
  auto la = mn_rows_idx_w8([=](int k) { return clamp_idx(sload_i32(row_token + off, k), T_); },
                           [=](int t) { return dyb + (int64_t)t * d * sizeof(bf16); }, cnt, m0, d);
  auto lb = mn_rows_w8([=](int k) { return wab + (int64_t)(off + k) * n * sizeof(bf16); }, cnt, n0, n);
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_w8(la, lb, (int)cdiv(cnt, Mma<bf16>::BK), acc, L, wm, bsub);
  bf16* out = dWd + (int64_t)e * d * n + (int64_t)m0 * n + n0;
  const int mrows = min(BM, d - m0), valid = min(BN, n - n0);
  epi_stage_w8(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v]; });
  __syncthreads();
  epi_store_rows<GEMM8_THREADS>(L, 0, [&](int r) { return out + (int64_t)r * n; }, mrows, BN, valid);
}

hipError_t launch_dw_down_gemm(const Shape& s, const PlanPtrs& p, const int32_t* order, const void* dY,
                               const void* wA, void* dW_down, hipStream_t st) {
  const int MT = (int)cdiv(s.d, BM), NT = (int)cdiv(s.n, BN);
  const int grid = grid8((int64_t)s.E * MT * NT);
  if (s.bf16)
    k_dw_down_w8<<<grid, GEMM8_THREADS, 0, st>>>(p.expert_off, order, p.row_token, (const bf16*)dY, (const bf16*)wA,
                                                 (bf16*)dW_down, (int)s.d, (int)s.n, s.E, MT, NT, (int)s.T);
  else
    k_dw_down<float><<<grid, GEMM_THREADS, 0, st>>>(p.expert_off, order, p.row_token, (const float*)dY,
                                                    (const float*)wA, (float*)dW_down, (int)s.d,
                                                    (int)s.n, s.E, MT, NT, (int)s.T);
  return hipGetLastError();
}

template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_dw_gu(
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ order, const int32_t* __restrict__ row_token,
    const T* __restrict__ dH, const T* __restrict__ X, T* __restrict__ dWg, T* __restrict__ dWu,
    int d, int n, int E, int MT, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  if (lin / per >= E) return;
  const int e = order[lin / per];
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int off = expert_off[e];
  const int cnt = expert_off[e + 1] - off;
  const char* dhb = reinterpret_cast<const char*>(dH) + m0 * sizeof(T);
  const char* xb = reinterpret_cast<const char*>(X) + n0 * sizeof(T);
  auto la = mn_rows<T>([=](int k) { return dhb + (int64_t)(off + k) * 2 * n * sizeof(T); }, cnt, m0, 2 * n);
  auto lb = mn_rows_idx<T>([=](int k) { return clamp_idx(sload_i32(row_token + off, k), T_); },
                          [=](int t) { return xb + (int64_t)t * d * sizeof(T); }, cnt, n0, d);
  WaveAcc acc;
  gemm_mainloop<T>(la, lb, (int)cdiv(cnt, Mma<T>::BK), acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  const int mrows = min(BM, 2 * n - m0), valid = min(BN, d - n0);
  auto row_ptr = [&](int r) -> T* {
    const int m = m0 + r;
    return (m < n ? dWg + ((int64_t)e * n + m) * d : dWu + ((int64_t)e * n + (m - n)) * d) + n0;
  };
  if constexpr (sizeof(T) == 2) {
    epi_stage_bf16(L, wm, [&](int j) { return bsub_plain(wn, j); },
                   [&](int i, int j, int v) { return acc.c[i][j][v]; });
    __syncthreads();
    epi_store_rows(L, 0, [&](int r) { return reinterpret_cast<bf16*>(row_ptr(r)); }, mrows, BN, valid);
  } else {
    epi_store_direct(wm, wn, acc, valid, mrows, row_ptr);
  }
}

// bf16 dW_gate | dW_up on the eight-wave engine (same tiles, operands and bits as k_dw_gu).
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_dw_gu_w8(
    const int32_t* __restrict__ expert_off, const int32_t* __restrict__ order, const int32_t* __restrict__ row_token,
    const bf16* __restrict__ dH, const bf16* __restrict__ X, bf16* __restrict__ dWg, bf16* __restrict__ dWu,
    int d, int n, int E, int MT, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  if (lin / per >= E) return;
  const int e = order[lin / per];
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int off = expert_off[e];
  const int cnt = expert_off[e + 1] - off;
  const char* dhb = reinterpret_cast<const char*>(dH) + m0 * sizeof(bf16);
  const char* xb = reinterpret_cast<const char*>(X) + n0 * sizeof(bf16);
  auto la = mn_rows_w8([=](int k) { return dhb + (int64_t)(off + k) * 2 * n * sizeof(bf16); }, cnt, m0, 2 * n);
  auto lb = mn_rows_idx_w8([=](int k) { return clamp_idx(sload_i32(row_token + off, k), T_); },
                           [=](int t) { return xb + (int64_t)t * d * sizeof(bf16); }, cnt, n0, d);
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_w8(la, lb, (int)cdiv(cnt, Mma<bf16>::BK), acc, L, wm, bsub);
  const int mrows = min(BM, 2 * n - m0), valid = min(BN, d - n0);
  epi_stage_w8(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v]; });
  __syncthreads();
  epi_store_rows<GEMM8_THREADS>(L, 0, [&](int r) -> bf16* {
    const int m = m0 + r;
    return (m < n ? dWg + ((int64_t)e * n + m) * d : dWu + ((int64_t)e * n + (m - n)) * d) + n0;
  }, mrows, BN, valid);
}

hipError_t launch_dw_gu_gemm(const Shape& s, const PlanPtrs& p, const int32_t* order, const void* dH,
                             const void* X, void* dW_gate, void* dW_up, hipStream_t st) {
  const int MT = (int)cdiv(2 * s.n, BM), NT = (int)cdiv(s.d, BN);
  const int grid = grid8((int64_t)s.E * MT * NT);
  if (s.bf16)
    k_dw_gu_w8<<<grid, GEMM8_THREADS, 0, st>>>(p.expert_off, order, p.row_token, (const bf16*)dH, (const bf16*)X,
                                               (bf16*)dW_gate, (bf16*)dW_up, (int)s.d, (int)s.n, s.E, MT, NT,
                                               (int)s.T);
  else
    k_dw_gu<float><<<grid, GEMM_THREADS, 0, st>>>(p.expert_off, order, p.row_token, (const float*)dH,
                                                  (const float*)X, (float*)dW_gate, (float*)dW_up,
                                                  (int)s.d, (int)s.n, s.E, MT, NT, (int)s.T);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Router backward fused with the dX gather-sum; one wave per token (4 tokens per block).
//   dS_r = sum over column tiles of dS_part;  s = sum_r w_r dS_r;  dL_r = w_r (dS_r - s)
//   dLogits[t][:] = dL on the token's experts, 0 elsewhere (dLop: the same row in the GEMM dtype,
//   padded to E_pad columns, the operand of the router weight gradient)
//   dX[t] = sum_r dX_perm[r] + dL_r W_r[e_r]      (rows in ascending expert order)
// ---------------------------------------------------------------------------------------------
// The expert of row r: a binary search over the block's LDS copy of expert_off.
__device__ __forceinline__ int expert_of_row(const int32_t* soff, int E, int r) {
  int lo = 0, hi = E;  // soff[lo] <= r < soff[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (soff[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

template <typename T, int CPL, int RB>
__global__ __launch_bounds__(256) void k_router_bwd(
    const int32_t* __restrict__ tok_off, const int32_t* __restrict__ tok_row,
    const int32_t* __restrict__ expert_off, const float* __restrict__ row_w,
    const float* __restrict__ dS_part, int ntiles, int64_t R_max, const T* __restrict__ dXp,
    const T* __restrict__ Wr, float* __restrict__ dS, float* __restrict__ dLogits,
    T* __restrict__ dLop, int E_pad, T* __restrict__ dX, int T_, int d, int E) {
  // per wave: the dense dL row [E_pad], the token's rows and their experts (at most E of each);
  // per block: expert_off [E + 1]
  extern __shared__ char rb_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  int* soff = reinterpret_cast<int*>(rb_lds) + (size_t)4 * 3 * E_pad;
  for (int e = threadIdx.x; e <= E; e += 256) soff[e] = expert_off[e];
  __syncthreads();
  if (t >= T_) return;
  const int base = tok_off[t], cnt = tok_off[t + 1] - base;
  float* sdl = reinterpret_cast<float*>(rb_lds) + (size_t)wave * 3 * E_pad;
  int* srow = reinterpret_cast<int*>(sdl + E_pad);
  int* sexp = srow + E_pad;
  for (int e = lane; e < E_pad; e += 64) sdl[e] = 0.0f;
  // pass 1: s = sum_r w_r dS_r; a lane keeps its first row's index, dS and weight for pass 2
  const int rmax = (int)R_max;
  auto row_ds = [&](int i, int& r, float& ds, float& w) {
    r = clamp_idx(tok_row[base + i], rmax);
    ds = 0.0f;
    for (int q = 0; q < ntiles; ++q) ds += dS_part[(int64_t)q * R_max + r];
    w = row_w[r];
  };
  int r0 = 0;
  float ds0 = 0.0f, w0 = 0.0f;
  if (lane < cnt) row_ds(lane, r0, ds0, w0);
  float part = w0 * ds0;
  for (int i = lane + 64; i < cnt; i += 64) {
    int r;
    float ds, w;
    row_ds(i, r, ds, w);
    part += w * ds;
  }
  const float ssum = wave_sum(part);
  // pass 2: dL per row, dS out, dense dL row in LDS; each row's expert resolved once
  auto put = [&](int i, int r, float ds, float w) {
    dS[r] = ds;
    const int e = expert_of_row(soff, E, r);
    sdl[e] = w * (ds - ssum);
    srow[i] = r;
    sexp[i] = e;
  };
  if (lane < cnt) put(lane, r0, ds0, w0);
  for (int i = lane + 64; i < cnt; i += 64) {
    int r;
    float ds, w;
    row_ds(i, r, ds, w);
    put(i, r, ds, w);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < E_pad; e += 64) {
    const float v = sdl[e];
    if (e < E) dLogits[(int64_t)t * E + e] = v;
    if (dLop) dLop[(int64_t)t * E_pad + e] = from_f32<T>(v);
  }
  // dX[t]: a lane owns CPL 16-byte column chunks (lane + 64 j) of a pass over the row; the
  // token's rows are taken RB at a time, and every dX_perm and W_r chunk of a batch is requested
  // before any is used, so a wave reads whole rows at once.  Rows are added in ascending expert
  // order.
  constexpr int VEC = 16 / sizeof(T);
  const int nch = d / VEC;
  for (int c0 = 0; c0 < nch; c0 += 64 * CPL) {
    float acc[CPL][VEC];
#pragma unroll
    for (int j = 0; j < CPL; ++j)
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[j][k] = 0.0f;
    bool ok[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) ok[j] = c0 + lane + 64 * j < nch;
    for (int i = 0; i < cnt; i += RB) {
      u32x4 v[RB][CPL], wv[RB][CPL];
      float dl[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const bool live = i + q < cnt;
        const int r = live ? srow[i + q] : 0;
        const int e = live ? sexp[i + q] : 0;
        dl[q] = live ? sdl[e] : 0.0f;
        const int64_t c = (int64_t)(c0 + lane) * VEC;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          v[q][j] = (live && ok[j]) ? ld16_nt(dXp + (int64_t)r * d + c + 64 * j * VEC) : u32x4{0u, 0u, 0u, 0u};
          wv[q][j] = (live && ok[j] && Wr) ? ld16(Wr + (int64_t)e * d + c + 64 * j * VEC) : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        if (i + q >= cnt) break;  // (uniform) the batch's rows past the token's last one add nothing
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          float f[VEC], w[VEC];
          unpack16<T>(v[q][j], f);
          unpack16<T>(wv[q][j], w);
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[j][k] += f[k] + dl[q] * w[k];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (ok[j]) st16(dX + (int64_t)t * d + (int64_t)(c0 + lane + 64 * j) * VEC, pack16<T>(acc[j]));
  }
}

template <typename T, int CPL, int RB>
static void router_bwd_for(const Shape& s, const PlanPtrs& p, const float* dS_part, int ntiles, const void* dX_perm,
                           const void* W_r, float* dS, float* dLogits, void* dLop, int E_pad, void* dX,
                           hipStream_t st) {
  const int grid = (int)cdiv(s.T, 4);
  const size_t lds = ((size_t)4 * 3 * E_pad + s.E + 1) * sizeof(float);  // <= 53 KiB for E <= 1024
  k_router_bwd<T, CPL, RB><<<grid, 256, lds, st>>>(p.tok_off, p.tok_row, p.expert_off, p.row_w, dS_part, ntiles,
                                                   s.R_max, static_cast<const T*>(dX_perm), static_cast<const T*>(W_r),
                                                   dS, dLogits, static_cast<T*>(dLop), E_pad, static_cast<T*>(dX),
                                                   (int)s.T, (int)s.d, s.E);
}

hipError_t launch_router_bwd(const Shape& s, const PlanPtrs& p, const float* dS_part, int ntiles,
                             const void* dX_perm, const void* W_r, float* dS, float* dLogits,
                             void* dLop, int E_pad, void* dX, hipStream_t st) {
  // chunks per lane: the whole row in one pass up to 4 * 64 16-byte chunks, else passes of that
  const int64_t nch = s.d / (s.bf16 ? 8 : 4);
#define MOE_RBWD(TT)                                                                                    \
  if (nch <= 64) router_bwd_for<TT, 1, 8>(s, p, dS_part, ntiles, dX_perm, W_r, dS, dLogits, dLop, E_pad, dX, st); \
  else if (nch <= 128) router_bwd_for<TT, 2, 4>(s, p, dS_part, ntiles, dX_perm, W_r, dS, dLogits, dLop, E_pad, dX, st); \
  else if (nch <= 192) router_bwd_for<TT, 3, 2>(s, p, dS_part, ntiles, dX_perm, W_r, dS, dLogits, dLop, E_pad, dX, st); \
  else router_bwd_for<TT, 4, 2>(s, p, dS_part, ntiles, dX_perm, W_r, dS, dLogits, dLop, E_pad, dX, st);
  if (s.bf16) { MOE_RBWD(bf16) } else { MOE_RBWD(float) }
#undef MOE_RBWD
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Router weight gradient dW_r[e][c] = sum_t dL[t][e] X[t][c]  (M = E, N = d, K = T).  The token
// range is split into S contiguous slices so that the few output tiles still fill the chip in one
// round (S * tiles <= 256 workgroups, one per CU); each slice writes fp32 partials, four
// consecutive columns per 16-byte store, and a second kernel sums the slices in a fixed order.
// ---------------------------------------------------------------------------------------------
struct DwrPlan {
  int MT, NT, S, TS;  // tiles, slices, tokens per slice (multiple of the stage depth)
};
static DwrPlan dwr_plan(const Shape& s) {
  DwrPlan q;
  q.MT = (int)cdiv(s.E, BM);
  q.NT = (int)cdiv(s.d, BN);
  const int bk = s.bf16 ? Mma<bf16>::BK : Mma<float>::BK;
  const int tiles = q.MT * q.NT;
  int S = 256 / tiles;
  const int max_s = (int)cdiv(s.T, bk);
  if (S > max_s) S = max_s;
  if (S > 64) S = 64;
  if (S < 1) S = 1;
  q.TS = (int)(cdiv(cdiv(s.T, S), bk) * bk);
  q.S = (int)cdiv(s.T, q.TS);
  return q;
}

size_t dwr_workspace_bytes(const Shape& s) {
  const DwrPlan q = dwr_plan(s);
  return q.S > 1 ? (size_t)q.S * s.E * s.d * sizeof(float) : 0;
}

template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_dwr(
    const T* __restrict__ dLop, int E_pad, const T* __restrict__ X, float* __restrict__ part,
    T* __restrict__ dWr, int T_, int d, int E, int MT, int NT, int S, int TS) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  const int sl = lin / per;
  if (sl >= S) return;
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int t0 = sl * TS;
  const int klen = min(TS, T_ - t0);
  const char* ab = reinterpret_cast<const char*>(dLop) + m0 * sizeof(T);
  const char* xb = reinterpret_cast<const char*>(X) + n0 * sizeof(T);
  auto la = mn_rows<T>([=](int k) { return ab + (int64_t)(t0 + k) * E_pad * sizeof(T); }, klen, m0, E_pad);
  auto lb = mn_rows<T>([=](int k) { return xb + (int64_t)(t0 + k) * d * sizeof(T); }, klen, n0, d);
  WaveAcc acc;
  gemm_mainloop<T>(la, lb, (int)cdiv(klen, Mma<T>::BK), acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  if (S == 1) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int c = n0 + bsub_plain(wn, j) + acc_n(v);
        if (c >= d) continue;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + acc_m(wm, i);
          if (m < E) dWr[(int64_t)m * d + c] = from_f32<T>(acc.c[i][j][v]);
        }
      }
    return;
  }
  // partials: a lane's four accumulators v = 4q .. 4q + 3 are consecutive columns (d is a
  // multiple of 64, so c < d implies c + 3 < d)
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = n0 + bsub_plain(wn, j) + acc_n(4 * q);
      if (c >= d) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + acc_m(wm, i);
        if (m >= E) continue;
        const f32x4 v4 = {acc.c[i][j][4 * q], acc.c[i][j][4 * q + 1], acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3]};
        *reinterpret_cast<f32x4*>(part + ((int64_t)sl * E + m) * d + c) = v4;
      }
    }
}

// bf16 on the eight-wave engine (same tiles, slices and bits as k_dwr; the four-wave kernel's
// 256 accumulator registers left it reloading spilled registers inside the main loop).
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_dwr_w8(
    const bf16* __restrict__ dLop, int E_pad, const bf16* __restrict__ X, float* __restrict__ part,
    bf16* __restrict__ dWr, int T_, int d, int E, int MT, int NT, int S, int TS) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = MT * NT;
  const int sl = lin / per;
  if (sl >= S) return;
  int mt, nt;
  raster_tile(lin % per, MT, NT, mt, nt);
  const int m0 = mt * BM, n0 = nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int t0 = sl * TS;
  const int klen = min(TS, T_ - t0);
  const char* ab = reinterpret_cast<const char*>(dLop) + m0 * sizeof(bf16);
  const char* xb = reinterpret_cast<const char*>(X) + n0 * sizeof(bf16);
  auto la = mn_rows_w8([=](int k) { return ab + (int64_t)(t0 + k) * E_pad * sizeof(bf16); }, klen, m0, E_pad);
  auto lb = mn_rows_w8([=](int k) { return xb + (int64_t)(t0 + k) * d * sizeof(bf16); }, klen, n0, d);
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_w8_rows(la, lb, (int)cdiv(klen, Mma<bf16>::BK), acc, L, wm, bsub, E - m0);
  // a lane's accumulators v = 4q .. 4q + 3 are four consecutive columns (d is a multiple of 64,
  // so c < d implies c + 3 < d)
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = n0 + bsub(j) + acc_n(4 * q);
      if (c >= d) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + acc_m(wm, i);
        if (m >= E) continue;
        if (S == 1) {
          const u32x2 pk = {pack_bf16x2(acc.c[i][j][4 * q], acc.c[i][j][4 * q + 1]),
                            pack_bf16x2(acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3])};
          *reinterpret_cast<u32x2*>(dWr + (int64_t)m * d + c) = pk;
        } else {
          const f32x4 v4 = {acc.c[i][j][4 * q], acc.c[i][j][4 * q + 1], acc.c[i][j][4 * q + 2], acc.c[i][j][4 * q + 3]};
          *reinterpret_cast<f32x4*>(part + ((int64_t)sl * E + m) * d + c) = v4;
        }
      }
    }
}

// Sums the S slices in slice order, four consecutive outputs per thread (n is a multiple of 4);
// the slices' loads are issued eight at a time.
template <typename T>
__global__ __launch_bounds__(256) void k_dwr_reduce(const float* __restrict__ part, int S,
                                                    int64_t n, T* __restrict__ dWr) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
  int q = 0;
  for (; q + 8 <= S; q += 8) {
    f32x4 v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(part + (int64_t)(q + k) * n + i));
#pragma unroll
    for (int k = 0; k < 8; ++k) s += v[k];
  }
  for (; q < S; ++q) s += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(part + (int64_t)q * n + i));
#pragma unroll
  for (int k = 0; k < 4; ++k) dWr[i + k] = from_f32<T>(s[k]);
}

hipError_t launch_dwr_gemm(const Shape& s, const void* dLop, int E_pad, const void* X, void* dW_r,
                           void* ws, hipStream_t st) {
  const DwrPlan q = dwr_plan(s);
  const int grid = grid8((int64_t)q.S * q.MT * q.NT);
  float* part = static_cast<float*>(ws);
  const int64_t nout = (int64_t)s.E * s.d;
  if (s.bf16) {
    k_dwr_w8<<<grid, GEMM8_THREADS, 0, st>>>((const bf16*)dLop, E_pad, (const bf16*)X, part, (bf16*)dW_r,
                                             (int)s.T, (int)s.d, s.E, q.MT, q.NT, q.S, q.TS);
    if (q.S > 1) k_dwr_reduce<bf16><<<(int)cdiv(nout / 4, 256), 256, 0, st>>>(part, q.S, nout, (bf16*)dW_r);
  } else {
    k_dwr<float><<<grid, GEMM_THREADS, 0, st>>>((const float*)dLop, E_pad, (const float*)X, part,
                                                (float*)dW_r, (int)s.T, (int)s.d, s.E, q.MT, q.NT, q.S, q.TS);
    if (q.S > 1) k_dwr_reduce<float><<<(int)cdiv(nout / 4, 256), 256, 0, st>>>(part, q.S, nout, (float*)dW_r);
  }
  return hipGetLastError();
}

}  // namespace moe

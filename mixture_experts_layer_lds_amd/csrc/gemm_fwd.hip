// Forward GEMMs: router logits, grouped gate/up projection with the SwiGLU epilogue, grouped
// down projection.
//
// Pages: apxml.com "自定义核与核融合" steps 1 and 4 (gate scores; the experts' dense matmuls);
// SonicMoE page "Gather 与加载融合" (the grouped GEMM reads either packed rows or rows gathered
// by index during its operand load) and the kernel-comparison table (SwiGLU fused into the GEMM);
// apxml.com "条件参数加载" (only experts that received tokens have their weights read: the tile
// list holds no tile for an empty expert).
#include "gemm_core.h"
#include "internal.h"

namespace moe {

// The tile table of the grouped GEMMs (see find_group_tile): table[0..E] = exclusive scan of
// ceil(counts[e] / BM); table[E + 1 .. 2 E + 1] = the same without the light tails (a last m-tile
// of 1..BM/2 rows); table[2 E + 2] = the number of light tails, table[2 E + 3 ..] = their experts
// in ascending order.  With order non-null also order[E]: the experts by decreasing row count,
// ties to the lower id (the weight-gradient GEMMs' tile order), so that the backward gets both
// tables from one launch.  One block, E <= 1024.
__global__ __launch_bounds__(1024) void k_tile_offsets(const int32_t* __restrict__ counts, int E,
                                                       int32_t* __restrict__ table,
                                                       int32_t* __restrict__ order) {
  __shared__ int sh[3][16];
  __shared__ int c[1024];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ce = threadIdx.x < E ? counts[threadIdx.x] : 0;
  if (order && threadIdx.x < E) c[threadIdx.x] = ce;
  const int rem = ce % BM;
  const int light = (rem > 0 && rem <= BM / 2) ? 1 : 0;
  const int x[3] = {(ce + BM - 1) / BM, (ce + BM - 1) / BM - light, light};
  int inc[3] = {x[0], x[1], x[2]};
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const int y = __shfl_up(inc[q], o, 64);
      if (lane >= o) inc[q] += y;
    }
  if (lane == 63)
#pragma unroll
    for (int q = 0; q < 3; ++q) sh[q][wave] = inc[q];
  __syncthreads();
  int base[3] = {0, 0, 0}, tot[3] = {0, 0, 0};
  for (int w = 0; w < 16; ++w)
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      base[q] += (w < wave) ? sh[q][w] : 0;
      tot[q] += sh[q][w];
    }
  if ((int)threadIdx.x < E) {
    table[threadIdx.x] = base[0] + inc[0] - x[0];
    table[E + 1 + threadIdx.x] = base[1] + inc[1] - x[1];
    if (light) table[2 * E + 3 + base[2] + inc[2] - 1] = threadIdx.x;
  }
  if (threadIdx.x == 0) {
    table[E] = tot[0];
    table[2 * E + 1] = tot[1];
    table[2 * E + 2] = tot[2];
  }
  if (order && (int)threadIdx.x < E) {
    const int e = threadIdx.x;
    int rank = 0;
    for (int f = 0; f < E; ++f) rank += (c[f] > ce || (c[f] == ce && f < e)) ? 1 : 0;
    order[rank] = e;
  }
}

hipError_t launch_tile_offsets(const int32_t* counts, int E, int32_t* mtile_off, int32_t* order, hipStream_t st) {
  k_tile_offsets<<<1, 1024, 0, st>>>(counts, E, mtile_off, order);
  return hipGetLastError();
}

int64_t max_mtiles(int64_t R_max, int E) { return R_max / BM + E; }

static inline int grid8(int64_t n) { return (int)((n + 7) / 8 * 8); }

// ---------------------------------------------------------------------------------------------
// Router: logits[t][e] = sum_i X[t][i] W_r[e][i] + bias[e]   (fp32 out, direct stores).  fp32
// layers: k_router (four-wave engine); bf16: k_router_h below.
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_router(const T* __restrict__ X,
                                                           const T* __restrict__ Wr,
                                                           const float* __restrict__ bias,
                                                           float* __restrict__ logits, int T_, int d,
                                                           int E, int NT) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = lin / NT, nt = lin % NT;
  const int m0 = mt * BM, n0 = nt * BN;
  if (m0 >= T_) return;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)d * sizeof(T);
  auto la = k_rows<T>([&](int i) -> const char* {
    return m0 + i < T_ ? reinterpret_cast<const char*>(X) + (m0 + i) * rowb : nullptr;
  });
  auto lb = k_rows<T>([&](int i) -> const char* {
    return n0 + i < E ? reinterpret_cast<const char*>(Wr) + (n0 + i) * rowb : nullptr;
  });
  WaveAcc acc;
  gemm_mainloop<T, true>(la, lb, d / Mma<T>::BK, acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  // a lane's accumulators v = 4q .. 4q + 3 are four consecutive experts of one token: one 16-byte
  // store when the logits rows keep them aligned (E % 4 == 0), else four 4-byte stores
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + bsub_plain(wn, j) + acc_n(4 * q);
      if (n >= E) continue;
      f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias) {
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = n + u < E ? bias[n + u] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + acc_m(wm, i);
        if (m >= T_) continue;
        float* o = logits + (int64_t)m * E + n;
        const f32x4 v4 = {acc.c[i][j][4 * q] + b[0], acc.c[i][j][4 * q + 1] + b[1], acc.c[i][j][4 * q + 2] + b[2],
                          acc.c[i][j][4 * q + 3] + b[3]};
        if ((E & 3) == 0) {
          *reinterpret_cast<f32x4*>(o) = v4;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (n + u < E) o[u] = v4[u];
        }
      }
    }
}

// bf16 router GEMM on the half-width engine: tile 256 tokens x 128 experts (the four-wave
// 256 x 256 tile would leave half its columns empty at E = 128), two workgroups per CU.  With
// SK > 1 workgroup (tile, ks) reduces over columns ks d / SK .. (ks + 1) d / SK only: at E = 128 a
// layer of 32768 tokens has 128 tiles, which alone would leave half the CUs idle.
__global__ __launch_bounds__(GEMM_THREADS, 2) void k_router_h(const bf16* __restrict__ X, const bf16* __restrict__ Wr,
                                                              const float* __restrict__ bias,
                                                              float* __restrict__ logits, float* __restrict__ part,
                                                              int T_, int d, int E, int NT, int SK) {
  MOE_GEMM_LDS_H(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tiles = (int)cdiv(T_, BM) * NT;
  const int ks = lin / tiles, tl = lin % tiles;  // reduction slice, output tile
  if (ks >= SK) return;
  const int mt = tl / NT, nt = tl % NT;
  const int m0 = mt * BM, n0 = nt * HBN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)d * sizeof(bf16);
  const int klen = d / SK;
  const int64_t k0b = (int64_t)ks * klen * sizeof(bf16);
  KDmaH<4> la;
  la.init([&](int i) -> const char* {
    return m0 + i < T_ ? reinterpret_cast<const char*>(X) + (m0 + i) * rowb + k0b : nullptr;
  });
  KDmaH<2> lb;
  lb.init([&](int i) -> const char* {
    return n0 + i < E ? reinterpret_cast<const char*>(Wr) + (n0 + i) * rowb + k0b : nullptr;
  });
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_h<false>(la, lb, klen / Mma<bf16>::BK, acc, L_0, L_1, L_2, wm, bsub);
  float* dst = ks == 0 ? logits : part + (int64_t)(ks - 1) * T_ * E;
  // as in k_router: a lane's v = 4q .. 4q + 3 are four consecutive experts of one token
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = n0 + bsub(j) + acc_n(4 * q);
      if (n >= E) continue;
      f32x4 b = {0.0f, 0.0f, 0.0f, 0.0f};
      if (bias && ks == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = n + u < E ? bias[n + u] : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + acc_m(wm, i);
        if (m >= T_) continue;
        float* o = dst + (int64_t)m * E + n;
        const f32x4 v4 = {acc.c[i][j][4 * q] + b[0], acc.c[i][j][4 * q + 1] + b[1], acc.c[i][j][4 * q + 2] + b[2],
                          acc.c[i][j][4 * q + 3] + b[3]};
        if ((E & 3) == 0) {
          *reinterpret_cast<f32x4*>(o) = v4;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (n + u < E) o[u] = v4[u];
        }
      }
    }
}

// Slices of the router GEMM's reduction: enough that the tiles fill the 256 CUs, at most 4, and
// each slice a whole number of k-steps, at least two.
int router_split(const Shape& s) {
  if (!s.bf16) return 1;
  const int64_t tiles = cdiv(s.T, BM) * cdiv(s.E, HBN);
  constexpr int BK = Mma<bf16>::BK;
  int sk = 1;
  while (sk < 4 && tiles * sk < 256 && s.d % (2 * sk * BK) == 0 && s.d / (2 * sk) >= 2 * BK) sk *= 2;
  return sk;
}

size_t router_part_bytes(const Shape& s) { return (size_t)(router_split(s) - 1) * s.T * s.E * sizeof(float); }

hipError_t launch_router_gemm(const Shape& s, const void* X, const void* W_r, const float* bias,
                              float* logits, float* part, hipStream_t st) {
  if (s.bf16) {
    const int NT = (int)cdiv(s.E, HBN);
    const int SK = router_split(s);
    k_router_h<<<grid8(cdiv(s.T, BM) * NT * SK), GEMM_THREADS, 0, st>>>((const bf16*)X, (const bf16*)W_r, bias,
                                                                       logits, part, (int)s.T, (int)s.d, s.E, NT, SK);
  } else {
    const int NT = (int)cdiv(s.E, BN);
    k_router<float><<<grid8(cdiv(s.T, BM) * NT), GEMM_THREADS, 0, st>>>((const float*)X, (const float*)W_r, bias,
                                                                       logits, (int)s.T, (int)s.d, s.E, NT);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Gate/up projection.  Tile = 256 rows of one expert x 128 output columns j0..j0+127; the B tile
// stacks W_gate[e] rows j0..j0+127 over W_up[e] rows j0..j0+127, and wave column wn takes gate
// blocks wn*64 + {0, 32} (j = 0, 1) and the up blocks 128 + wn*64 + {0, 32} (j = 2, 3), so each
// lane holds G and U of the same (row, column) in accumulators j and j + 2.  Epilogue:
// A = silu(G) U in fp32, rounded once; optional H = [G | U].
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_up(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const T* __restrict__ A_in, int gathered,
    const T* __restrict__ Wg, const T* __restrict__ Wu, T* __restrict__ act, T* __restrict__ H,
    int d, int n, int E, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int nt = g.nt;
  const int j0 = nt * 128;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)d * sizeof(T);
  auto la = k_rows<T>([&](int i) -> const char* {
    if (i >= g.mrows) return nullptr;
    const int64_t src = gathered ? clamp_idx(row_token[g.m0 + i], T_) : (int64_t)(g.m0 + i);
    return reinterpret_cast<const char*>(A_in) + src * rowb;
  });
  const char* wg = reinterpret_cast<const char*>(Wg) + (int64_t)g.e * n * rowb;
  const char* wu = reinterpret_cast<const char*>(Wu) + (int64_t)g.e * n * rowb;
  auto lb = k_rows<T>([&](int i) -> const char* {
    const int j = j0 + (i & 127);
    if (j >= n) return nullptr;
    return (i < 128 ? wg : wu) + (int64_t)j * rowb;
  });
  WaveAcc acc;
  // B blocks j = 0, 1 are gate columns, j = 2, 3 the up columns of the same act columns
  gemm_mainloop<T, true>(la, lb, d / Mma<T>::BK, acc, L, wm, [&](int j) { return bsub_halved(wn, j); });
  const int valid = min(128, n - j0);
  if constexpr (sizeof(T) == 2) {
    auto silu_u = [&](int i, int j, int v) {
      const float gv = acc.c[i][j & 1][v], uv = acc.c[i][(j & 1) + 2][v];
      return gv * sigmoid_f32(gv) * uv;
    };
    auto colf = [&](int j) { return j < 2 ? bsub_halved(wn, j) : -1; };
    epi_stage_bf16(L, wm, colf, silu_u);
    __syncthreads();
    epi_store_bf16(L, 0, reinterpret_cast<bf16*>(act) + (int64_t)g.m0 * n + j0, n, g.mrows, 128, valid);
    if (H) {
      // G and U halves side by side in one staging tile: columns [0,128) G, [128,256) U
      __syncthreads();
      auto both = [&](int j) { return bsub_halved(wn, j); };
      epi_stage_bf16(L, wm, both, [&](int i, int j, int v) { return acc.c[i][j][v]; });
      __syncthreads();
      bf16* hb = reinterpret_cast<bf16*>(H) + (int64_t)g.m0 * 2 * n;
      epi_store_bf16(L, 0, hb + j0, 2 * n, g.mrows, 128, valid);
      epi_store_bf16(L, 128, hb + n + j0, 2 * n, g.mrows, 128, valid);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int ccol = bsub_halved(wn, j) + acc_n(v);  // act column within the tile
        if (ccol >= valid) continue;
        const int col = j0 + ccol;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = acc_m(wm, i);
          if (m >= g.mrows) continue;
          const int64_t r = g.m0 + m;
          const float gv = acc.c[i][j][v], uv = acc.c[i][j + 2][v];
          act[r * n + col] = from_f32<T>(gv * sigmoid_f32(gv) * uv);
          if (H) {
            H[r * 2 * n + col] = from_f32<T>(gv);
            H[r * 2 * n + n + col] = from_f32<T>(uv);
          }
        }
      }
  }
}

// bf16 gate/up on the eight-wave engine (same tiles, operands and bits as k_up; 4% faster on the
// fine-grained layer, where the down GEMM, K = n = 256, was 4% slower on it and stays on four
// waves): wave column wn
// takes gate block j = 0 at columns wn * 32 and up block j = 1 at 128 + wn * 32 of the stacked B
// tile, so G and U of one (row, column) again sit in the same lane.
__global__ __launch_bounds__(GEMM8_THREADS, 1) void k_up_w8(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const bf16* __restrict__ A_in, int gathered,
    const bf16* __restrict__ Wg, const bf16* __restrict__ Wu, bf16* __restrict__ act, bf16* __restrict__ H,
    int d, int n, int E, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int j0 = g.nt * 128;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int64_t rowb = (int64_t)d * sizeof(bf16);
  KDmaW8 la, lb;
  la.init([&](int i) -> const char* {
    if (i >= g.mrows) return nullptr;
    const int64_t src = gathered ? clamp_idx(row_token[g.m0 + i], T_) : (int64_t)(g.m0 + i);
    return reinterpret_cast<const char*>(A_in) + src * rowb;
  });
  const char* wg = reinterpret_cast<const char*>(Wg) + (int64_t)g.e * n * rowb;
  const char* wu = reinterpret_cast<const char*>(Wu) + (int64_t)g.e * n * rowb;
  lb.init([&](int i) -> const char* {
    const int j = j0 + (i & 127);
    if (j >= n) return nullptr;
    return (i < 128 ? wg : wu) + (int64_t)j * rowb;
  });
  auto bsub = [&](int j) { return j * 128 + wn * 32; };
  AccW8 acc;
  gemm_mainloop_w8_rows(la, lb, d / Mma<bf16>::BK, acc, L, wm, bsub, g.mrows);
  const int valid = min(128, n - j0);
  epi_stage_w8(L, wm, [&](int j) { return j == 0 ? wn * 32 : -1; }, [&](int i, int, int v) {
    const float gv = acc.c[i][0][v], uv = acc.c[i][1][v];
    return gv * sigmoid_f32(gv) * uv;
  });
  __syncthreads();
  bf16* ab = act + (int64_t)g.m0 * n + j0;
  epi_store_rows<GEMM8_THREADS>(L, 0, [&](int r) { return ab + (int64_t)r * n; }, g.mrows, 128, valid);
  if (H) {
    // G and U side by side in one staging tile: columns [0,128) G, [128,256) U
    __syncthreads();
    epi_stage_w8(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v]; });
    __syncthreads();
    bf16* hb = H + (int64_t)g.m0 * 2 * n;
    epi_store_rows<GEMM8_THREADS>(L, 0, [&](int r) { return hb + (int64_t)r * 2 * n + j0; }, g.mrows, 128, valid);
    epi_store_rows<GEMM8_THREADS>(L, 128, [&](int r) { return hb + (int64_t)r * 2 * n + n + j0; }, g.mrows, 128,
                                  valid);
  }
}

hipError_t launch_up_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                          const void* A_in, bool gathered, const void* W_gate, const void* W_up,
                          void* act, void* H, hipStream_t st) {
  const int NT = (int)cdiv(s.n, 128);
  const int grid = grid8(max_mtiles(s.R_max, s.E) * NT);
  if (s.bf16) {
    k_up_w8<<<grid, GEMM8_THREADS, 0, st>>>(mtile_off, p.expert_off, p.row_token, (const bf16*)A_in, gathered,
                                            (const bf16*)W_gate, (const bf16*)W_up, (bf16*)act, (bf16*)H, (int)s.d,
                                            (int)s.n, s.E, NT, (int)s.T);
    return hipGetLastError();
  }
  k_up<float><<<grid, GEMM_THREADS, 0, st>>>(mtile_off, p.expert_off, p.row_token, (const float*)A_in,
                                                      gathered, (const float*)W_gate, (const float*)W_up,
                                                      (float*)act, (float*)H, (int)s.d, (int)s.n, s.E, NT, (int)s.T);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------------
// Down projection: Y[r][c] = sum_j Act[r][j] W_down[e][c][j];  tile 256 rows x 256 columns of d on
// the four-wave engine (fp32 layers, and bf16 layers with long K; k_down_h below for short K).
// ---------------------------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_down(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const T* __restrict__ act, const T* __restrict__ Wd, T* __restrict__ Y, int d, int n, int E,
    int NT) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)n * sizeof(T);
  auto la = k_rows<T>([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(act) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wd) + (int64_t)g.e * d * rowb;
  auto lb = k_rows<T>([&](int i) -> const char* { return n0 + i < d ? wd + (int64_t)(n0 + i) * rowb : nullptr; });
  WaveAcc acc;
  gemm_mainloop<T, true>(la, lb, n / Mma<T>::BK, acc, L, wm, [&](int j) { return bsub_plain(wn, j); });
  const int valid = min(BN, d - n0);
  if constexpr (sizeof(T) == 2) {
    epi_stage_bf16(L, wm, [&](int j) { return bsub_plain(wn, j); },
                   [&](int i, int j, int v) { return acc.c[i][j][v]; });
    __syncthreads();
    epi_store_bf16(L, 0, reinterpret_cast<bf16*>(Y) + (int64_t)g.m0 * d + n0, d, g.mrows, BN, valid);
  } else {
    epi_store_direct(wm, wn, acc, valid, g.mrows, [&](int m) { return Y + (int64_t)(g.m0 + m) * d + n0; });
  }
}

// bf16 down projection on the half-width engine, for n <= DOWN_H_MAX_N: tile 256 rows x 128
// columns of d, two workgroups per CU (a tile has only n / 32 k-stages, so filling the ring and
// storing the R x d output are a large share of its time; the second workgroup's main loop runs
// beside them).  With long K the four-wave tile's operand reuse wins.
__global__ __launch_bounds__(GEMM_THREADS, 2) void k_down_h(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const bf16* __restrict__ act, const bf16* __restrict__ Wd, bf16* __restrict__ Y, int d, int n, int E,
    int NT) {
  MOE_GEMM_LDS_H(L);
  const int lin = xcd_remap<96>(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * HBN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = (int64_t)n * sizeof(bf16);
  KDmaH<4> la;
  la.init([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(act) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wd) + (int64_t)g.e * d * rowb;
  KDmaH<2> lb;
  lb.init([&](int i) -> const char* { return n0 + i < d ? wd + (int64_t)(n0 + i) * rowb : nullptr; });
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_h<false>(la, lb, n / Mma<bf16>::BK, acc, L_0, L_1, L_2, wm, bsub);
  bf16* out = Y + (int64_t)g.m0 * d + n0;
  epi_h([&](int i, int j, int v) { return acc.c[i][j][v]; }, L_0, L_1, L_2, wm, bsub,
        [&](int r) { return out + (int64_t)r * d; }, g.mrows, min(HBN, d - n0));
}

hipError_t launch_down_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                            const void* act, const void* W_down, void* Y, hipStream_t st) {
  if (s.bf16 && s.n <= DOWN_H_MAX_N) {
    const int NT = (int)cdiv(s.d, HBN);
    k_down_h<<<grid8(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, (const bf16*)act, (const bf16*)W_down, (bf16*)Y, (int)s.d, (int)s.n, s.E, NT);
  } else if (s.bf16) {
    const int NT = (int)cdiv(s.d, BN);
    k_down<bf16><<<grid8(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, (const bf16*)act, (const bf16*)W_down, (bf16*)Y, (int)s.d, (int)s.n, s.E, NT);
  } else {
    const int NT = (int)cdiv(s.d, BN);
    k_down<float><<<grid8(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, (const float*)act, (const float*)W_down, (float*)Y, (int)s.d, (int)s.n, s.E, NT);
  }
  return hipGetLastError();
}

}  // namespace moe

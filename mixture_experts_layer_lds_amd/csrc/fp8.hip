// FP8 expert FFN: per-row E4M3 quantisation and the grouped gate/up and down GEMMs on codes.
//
// Pages: apxml.com "硬件加速的考量", section "利用稀疏性和量化" / "量化" (weights and activations
// in low precision such as FP8: smaller experts, fewer bytes moved when the active experts are
// loaded, faster low-precision matrix units).  The pages fix no format or scaling; this path
// uses OCP FP8 E4M3 codes with one power-of-two scale per row of every operand (token rows of
// activations, output channels of weights): the smallest power of two s with max|row| / s <= 448.
// A power of two makes x / s exact, so the encoding (nearest code, ties to even) is decided the
// same way in any precision.
//
//   k_quant_fp8:  rows x K elements -> codes [rows][K] (uint8) and scales [rows] (fp32);
//   k_up_fp8 / k_up_fp8_h: act = silu(G) U with G, U = (Xq[rows] [Wg_q; Wu_q]^T) * s_x * s_w, gathered token
//                 rows as in the bf16 gate/up GEMM; act stored in bf16;
//   k_down_fp8 / k_down_fp8_h: Y = (act_q Wd_q^T) * s_a * s_d, stored in bf16.
// The GEMMs run the bf16 path's DMA ring and tile schedule with 64 one-byte elements per stage
// on v_mfma_scale_f32_32x32x64_f8f6f4 (fp32 accumulation of exact products); the scales are
// applied in the epilogue.
#include "gemm_core.h"
#include "internal.h"

namespace moe {

// One wave per row (four per workgroup).  rows_dev (optional) bounds the rows on the device.
// The codes come from the hardware conversion v_cvt_pk_fp8_f32 (two values per instruction;
// OCP E4M3, nearest with ties to the even code, subnormals kept), applied to x / s, which is
// exact because s is a power of two.
template <typename T>
__global__ __launch_bounds__(256) void k_quant_fp8(const T* __restrict__ src, int64_t rows, int K,
                                                   const int32_t* __restrict__ rows_dev, uint8_t* __restrict__ codes,
                                                   float* __restrict__ scales) {
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nrows = rows_dev ? (int64_t)rows_dev[0] : rows;
  if (row >= rows || row >= nrows) return;
  const T* s = src + row * K;
  float amax = 0.0f;
  for (int c = lane * VEC; c < K; c += 64 * VEC) {
    float f[8];
    unpack16<T>(ld16(s + c), f);
#pragma unroll
    for (int i = 0; i < VEC; ++i) amax = fmaxf(amax, fabsf(f[i]));
  }
  amax = wave_max(amax);
  int sexp = 0;
  if (amax > 0.0f) {
    int ex;
    const float fr = frexpf(amax, &ex);  // amax = fr 2^ex, fr in [0.5, 1)
    sexp = ex - 9 + (fr > 0.875f ? 1 : 0);
  }
  if (lane == 0) scales[row] = ldexpf(1.0f, sexp);
  uint8_t* o = codes + row * K;
  for (int c = lane * VEC; c < K; c += 64 * VEC) {
    float f[8];
    unpack16<T>(ld16(s + c), f);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < VEC; i += 4) {
      const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[i], -sexp), ldexpf(f[i + 1], -sexp), 0, false);
      w[i >> 2] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(f[i + 2], -sexp), ldexpf(f[i + 3], -sexp), lo, true);
    }
    if constexpr (VEC == 8) *reinterpret_cast<u32x2*>(o + c) = u32x2{w[0], w[1]};
    else *reinterpret_cast<uint32_t*>(o + c) = w[0];
  }
}

hipError_t launch_quant_fp8(const void* src, bool is_bf16, int64_t rows, int64_t K, const int32_t* rows_dev,
                            uint8_t* codes, float* scales, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (is_bf16)
    k_quant_fp8<bf16><<<grid, 256, 0, st>>>(static_cast<const bf16*>(src), rows, (int)K, rows_dev, codes, scales);
  else
    k_quant_fp8<float><<<grid, 256, 0, st>>>(static_cast<const float*>(src), rows, (int)K, rows_dev, codes, scales);
  return hipGetLastError();
}

// Four consecutive fp32 scales at p (16-byte aligned), or zeros past `valid` columns.
__device__ __forceinline__ f32x4 scales4(const float* p, bool ok) {
  return ok ? *reinterpret_cast<const f32x4*>(p) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
}

// ---------------------------------------------------------------------------------------------
// Gate/up: tile = 256 rows of one expert x 128 act columns j0 .. j0 + 127; the B tile stacks
// W_gate[e] rows j0 .. j0 + 127 over W_up[e] rows j0 .. j0 + 127 (halved block layout, so G and
// U of a (row, column) sit in accumulator blocks j and j + 2 of the same lane).
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_up_fp8(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const uint8_t* __restrict__ Xq, const float* __restrict__ sx,
    const uint8_t* __restrict__ Wgq, const float* __restrict__ sg, const uint8_t* __restrict__ Wuq,
    const float* __restrict__ su, bf16* __restrict__ act, int d, int n, int E, int NT, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int j0 = g.nt * 128;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = d;  // one byte per element
  KDma la, lb;
  la.init([&](int i) -> const char* {
    if (i >= g.mrows) return nullptr;
    return reinterpret_cast<const char*>(Xq) + (int64_t)clamp_idx(row_token[g.m0 + i], T_) * rowb;
  });
  const char* wg = reinterpret_cast<const char*>(Wgq) + (int64_t)g.e * n * rowb;
  const char* wu = reinterpret_cast<const char*>(Wuq) + (int64_t)g.e * n * rowb;
  lb.init([&](int i) -> const char* {
    const int j = j0 + (i & 127);
    if (j >= n) return nullptr;
    return (i < 128 ? wg : wu) + (int64_t)j * rowb;
  });
  WaveAcc acc;
  auto bsub = [&](int j) { return bsub_halved(wn, j); };
  gemm_mainloop_f8(la, lb, d / 64, acc, L, wm, bsub);
  const int valid = min(128, n - j0);
  // row scales of the wave's four row blocks (token rows) and column scales of its gate/up columns
  float srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    srow[i] = r < g.mrows ? sx[clamp_idx(row_token[g.m0 + r], T_)] : 0.0f;
  }
  f32x4 cg[2][4], cu[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = bsub(j) + acc_n(4 * q);
      const int64_t w = (int64_t)g.e * n + j0 + c;
      cg[j][q] = scales4(sg + w, c < valid);
      cu[j][q] = scales4(su + w, c < valid);
    }
  auto silu_u = [&](int i, int j, int v) {
    const float gv = acc.c[i][j & 1][v] * srow[i] * cg[j & 1][v >> 2][v & 3];
    const float uv = acc.c[i][(j & 1) + 2][v] * srow[i] * cu[j & 1][v >> 2][v & 3];
    return gv * sigmoid_f32(gv) * uv;
  };
  epi_stage_bf16(L, wm, [&](int j) { return j < 2 ? bsub(j) : -1; }, silu_u);
  __syncthreads();
  epi_store_bf16(L, 0, act + (int64_t)g.m0 * n + j0, n, g.mrows, 128, valid);
}

// The same on the half-width engine, for d <= UP_H_MAX_D_FP8 (at most 32 fp8 k-stages per tile,
// where the second workgroup per CU hides the ring fill and the epilogue; with longer K the
// four-wave tile's operand reuse wins): tile 256 rows x 64 act columns (B: W_gate rows j0 .. j0 + 63
// over W_up rows j0 .. j0 + 63; block j of wave column wn at j * 64 + wn * 32, so G and U of a
// (row, column) sit in accumulator blocks 0 and 1 of one lane), two workgroups per CU.
constexpr int UP_H_MAX_D_FP8 = 2048;
constexpr int UP8H_COLS = 64;
constexpr int UP8H_ROW = UP8H_COLS * 2 + 16;  // bf16 staging pitch
constexpr int UP8H_ROWS = H_SLOT / UP8H_ROW;   // staging rows per slot (170; two slots hold 256)
static_assert(2 * UP8H_ROWS >= BM, "act staging fits two slots");

__global__ __launch_bounds__(GEMM_THREADS, 2) void k_up_fp8_h(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const uint8_t* __restrict__ Xq, const float* __restrict__ sx,
    const uint8_t* __restrict__ Wgq, const float* __restrict__ sg, const uint8_t* __restrict__ Wuq,
    const float* __restrict__ su, bf16* __restrict__ act, int d, int n, int E, int NT, int T_) {
  MOE_GEMM_LDS_H(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int j0 = g.nt * UP8H_COLS;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = d;  // one byte per element
  KDmaH<4> la;
  la.init([&](int i) -> const char* {
    if (i >= g.mrows) return nullptr;
    return reinterpret_cast<const char*>(Xq) + (int64_t)clamp_idx(row_token[g.m0 + i], T_) * rowb;
  });
  const char* wg = reinterpret_cast<const char*>(Wgq) + (int64_t)g.e * n * rowb;
  const char* wu = reinterpret_cast<const char*>(Wuq) + (int64_t)g.e * n * rowb;
  KDmaH<2> lb;
  lb.init([&](int i) -> const char* {
    const int j = j0 + (i & 63);
    if (j >= n) return nullptr;
    return (i < 64 ? wg : wu) + (int64_t)j * rowb;
  });
  auto bsub = [&](int j) { return j * 64 + wn * 32; };
  AccW8 acc;
  gemm_mainloop_h<true>(la, lb, d / 64, acc, L_0, L_1, L_2, wm, bsub);
  const int valid = min(UP8H_COLS, n - j0);
  float srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    srow[i] = r < g.mrows ? sx[clamp_idx(row_token[g.m0 + r], T_)] : 0.0f;
  }
  f32x4 cg[4], cu[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = wn * 32 + acc_n(4 * q);
    const int64_t w = (int64_t)g.e * n + j0 + c;
    cg[q] = scales4(sg + w, c < valid);
    cu[q] = scales4(su + w, c < valid);
  }
  auto srow_ptr = [&](int r) { return (r < UP8H_ROWS ? L_0 + r * UP8H_ROW : L_1 + (r - UP8H_ROWS) * UP8H_ROW); };
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    char* row = srow_ptr(acc_m(wm, i));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float gv = acc.c[i][0][4 * q + u] * srow[i] * cg[q][u];
        const float uv = acc.c[i][1][4 * q + u] * srow[i] * cu[q][u];
        a[u] = gv * sigmoid_f32(gv) * uv;
      }
      const u32x2 pk = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
      *reinterpret_cast<u32x2*>(row + (wn * 32 + acc_n(4 * q)) * 2) = pk;
    }
  }
  __syncthreads();
  bf16* out = act + (int64_t)g.m0 * n + j0;
  u32x4 v[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int c = threadIdx.x + b * GEMM_THREADS;
    v[b] = *reinterpret_cast<const u32x4*>(srow_ptr(c >> 3) + (c & 7) * 16);
  }
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int c = threadIdx.x + b * GEMM_THREADS;
    const int r = c >> 3, ch = c & 7;
    if (r < g.mrows && ch * 8 < valid) st16_nt(out + (int64_t)r * n + ch * 8, v[b]);
  }
}

// ---------------------------------------------------------------------------------------------
// Down: Y[r][c] = (sum_j act_q[r][j] Wd_q[e][c][j]) s_a[r] s_d[e][c].
//   k_down_fp8:   tile 256 rows x 256 columns of d on the four-wave engine;
//   k_down_fp8_h: tile 256 rows x 128 columns on the half-width engine, two workgroups per CU,
//                 for short K (n <= DOWN_H_MAX_N_FP8): a tile's ring fill and bf16 output stores
//                 are then a large share of its time, and the second workgroup's MFMAs run
//                 beside them.  With long K the four-wave tile's operand reuse wins.
// ---------------------------------------------------------------------------------------------
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_down_fp8(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const uint8_t* __restrict__ Aq, const float* __restrict__ sa, const uint8_t* __restrict__ Wdq,
    const float* __restrict__ sd, bf16* __restrict__ Y, int d, int n, int E, int NT) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = n;
  KDma la, lb;
  la.init([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(Aq) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wdq) + (int64_t)g.e * d * rowb;
  lb.init([&](int i) -> const char* { return n0 + i < d ? wd + (int64_t)(n0 + i) * rowb : nullptr; });
  WaveAcc acc;
  auto bsub = [&](int j) { return bsub_plain(wn, j); };
  gemm_mainloop_f8(la, lb, n / 64, acc, L, wm, bsub);
  const int valid = min(BN, d - n0);
  float srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    srow[i] = r < g.mrows ? sa[g.m0 + r] : 0.0f;
  }
  f32x4 cs[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = bsub(j) + acc_n(4 * q);
      cs[j][q] = scales4(sd + (int64_t)g.e * d + n0 + c, c < valid);
    }
  epi_stage_bf16(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v] * srow[i] * cs[j][v >> 2][v & 3]; });
  __syncthreads();
  epi_store_bf16(L, 0, Y + (int64_t)g.m0 * d + n0, d, g.mrows, BN, valid);
}


__global__ __launch_bounds__(GEMM_THREADS, 2) void k_down_fp8_h(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const uint8_t* __restrict__ Aq, const float* __restrict__ sa, const uint8_t* __restrict__ Wdq,
    const float* __restrict__ sd, bf16* __restrict__ Y, int d, int n, int E, int NT) {
  MOE_GEMM_LDS_H(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * HBN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t rowb = n;
  KDmaH<4> la;
  la.init([&](int i) -> const char* {
    return i < g.mrows ? reinterpret_cast<const char*>(Aq) + (int64_t)(g.m0 + i) * rowb : nullptr;
  });
  const char* wd = reinterpret_cast<const char*>(Wdq) + (int64_t)g.e * d * rowb;
  KDmaH<2> lb;
  lb.init([&](int i) -> const char* { return n0 + i < d ? wd + (int64_t)(n0 + i) * rowb : nullptr; });
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_h<true>(la, lb, n / 64, acc, L_0, L_1, L_2, wm, bsub);
  const int valid = min(HBN, d - n0);
  float srow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    srow[i] = r < g.mrows ? sa[g.m0 + r] : 0.0f;
  }
  f32x4 cs[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = bsub(j) + acc_n(4 * q);
      cs[j][q] = scales4(sd + (int64_t)g.e * d + n0 + c, c < valid);
    }
  bf16* out = Y + (int64_t)g.m0 * d + n0;
  epi_h([&](int i, int j, int v) { return acc.c[i][j][v] * srow[i] * cs[j][v >> 2][v & 3]; }, L_0, L_1, L_2, wm,
        bsub, [&](int r) { return out + (int64_t)r * d; }, g.mrows, valid);
}

// =============================================================================================
// Block-scaled FP8: E4M3 (FMT 0) or E5M2 (FMT 1) codes with one E8M0 scale byte per 32 consecutive
// elements along K.  The scale of a block is the smallest power of two s with max|block| / s <=
// the format's largest finite value (448 or 57344), s = 1 for an all-zero block, kept within
// 2^-127 .. 2^127; the byte is log2(s) + 127.  Scales are stored group-major, [ceil(K / 128)]
// [rows][4 bytes]: block b of row r is byte (b / 4) * rows * 4 + r * 4 + b % 4 (the layout the
// GEMMs load 64 rows of in one 256-byte access); bytes of blocks past K / 32 are unspecified.
// =============================================================================================
// log2 of the block scale for a block maximum `amax` (format exponent E: 448 = 0.875 2^9,
// 57344 = 0.875 2^16).
template <int FMT>
__device__ __forceinline__ int mx_exponent(float amax) {
  constexpr int E = FMT == 0 ? 9 : 16;
  if (!(amax > 0.0f)) return 0;
  int ex;
  const float fr = frexpf(amax, &ex);  // amax = fr 2^ex, fr in [0.5, 1)
  const int k = ex - E + (fr > 0.875f ? 1 : 0);
  return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// Two fp32 values (already divided by the block scale) to codes, packed into bytes 0-1 (hi =
// false) or 2-3 of `old`: the hardware conversions round to the nearest code, ties to even.
template <int FMT, bool HI>
__device__ __forceinline__ int mx_cvt2(float a, float b, int old) {
  if constexpr (FMT == 0) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}

// One wave per row, one lane per 32-element block (lanes stride over the row's blocks).
template <typename T, int FMT>
__global__ __launch_bounds__(256) void k_quant_mx(const T* __restrict__ src, int64_t rows, int K,
                                                  uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  constexpr int VEC = 16 / sizeof(T);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int nb = K / 32;
  for (int b = lane; b < nb; b += 64) {
    const T* p = src + row * K + b * 32;
    float f[32];
#pragma unroll
    for (int c = 0; c < 32; c += VEC) unpack16<T>(ld16(p + c), f + c);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
    const int k = mx_exponent<FMT>(amax);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const int lo = mx_cvt2<FMT, false>(ldexpf(f[i], -k), ldexpf(f[i + 1], -k), 0);
      w[i >> 2] = (uint32_t)mx_cvt2<FMT, true>(ldexpf(f[i + 2], -k), ldexpf(f[i + 3], -k), lo);
    }
    uint8_t* o = codes + row * K + b * 32;
    *reinterpret_cast<u32x4*>(o) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4*>(o + 16) = u32x4{w[4], w[5], w[6], w[7]};
    scales[((int64_t)(b >> 2) * rows + row) * 4 + (b & 3)] = (uint8_t)(k + 127);
  }
}

int64_t mx_scale_bytes(int64_t rows, int64_t K) { return (K + 127) / 128 * rows * 4; }

hipError_t launch_quant_mx(const void* src, bool is_bf16, int fmt, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
#define MOE_QMX(TT, F) k_quant_mx<TT, F><<<grid, 256, 0, st>>>(static_cast<const TT*>(src), rows, (int)K, codes, scales)
  if (is_bf16) { if (fmt == 0) MOE_QMX(bf16, 0); else MOE_QMX(bf16, 1); }
  else { if (fmt == 0) MOE_QMX(float, 0); else MOE_QMX(float, 1); }
#undef MOE_QMX
  return hipGetLastError();
}

// The token scales in routed-row order, so that a gate/up tile's rows have contiguous scale words:
// sxp[g][r] = sx[g][row_token[r]] for the rows r < R of the plan (4-byte words, groups of d).
__global__ __launch_bounds__(256) void k_gather_mx_scales(const uint32_t* __restrict__ sx,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ meta, int64_t T,
                                                          int64_t R_max, int groups, uint32_t* __restrict__ sxp) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= meta[0] || r >= R_max) return;
  const int64_t t = clamp_idx(row_token[r], (int)T);
  for (int g = 0; g < groups; ++g) sxp[g * R_max + r] = sx[g * T + t];
}

// Gate/up with block scales on the half-width engine: tile 256 rows x 64 act columns (B: W_gate
// rows j0 .. j0 + 63 over W_up rows j0 .. j0 + 63, as k_up_fp8_h).  The epilogue forms
// act = silu(G) U, rounds it to bf16 (stored too if `act` is given), and quantises it in place:
// wave column wn holds act columns j0 + 32 wn .. + 31 -- one scale block -- of its rows, split
// between lanes l and l + 32, so a block's maximum is one exchange between them.  Codes are staged
// in LDS and stored in 16-byte chunks; scale bytes are stored by lanes 0-31.
constexpr int MXC_ROW = UP8H_COLS + 16;  // code staging pitch (bytes)

template <int FMT>
__global__ __launch_bounds__(GEMM_THREADS, 2) void k_up_mx_h(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ sx,
    const uint8_t* __restrict__ Wgq, const uint8_t* __restrict__ sg, const uint8_t* __restrict__ Wuq,
    const uint8_t* __restrict__ su, bf16* __restrict__ act, uint8_t* __restrict__ act_q,
    uint8_t* __restrict__ sact, int d, int n, int E, int NT, int64_t R_max, int T_) {
  MOE_GEMM_LDS_HMX(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int j0 = g.nt * UP8H_COLS;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  // rows past the tile's valid ones read the last valid row (never stored); the code offsets of
  // gathered rows fit in 32 bits (checked on the host: T * d < 2^32).  sx: the token scales in
  // routed-row order (k_gather_mx_scales), planes of R_max rows.
  auto rowi = [&](int i) { return g.m0 + min(i, g.mrows - 1); };
  KDmaHU<4> la;
  la.init([&](int) { return reinterpret_cast<const char*>(Xq); },
          [&](int i) { return (uint32_t)clamp_idx(row_token[rowi(i)], T_) * (uint32_t)d; });
  ScaleDmaH<4> sa;
  sa.init([&](int) { return reinterpret_cast<const char*>(sx); }, R_max * 4, [&](int i) { return (uint32_t)rowi(i) * 4u; });
  // B rows 0-63: W_gate rows j0 .. j0 + 63, rows 64-127: W_up (n is a multiple of 64: all valid)
  const int64_t wrow0 = (int64_t)g.e * n + j0;
  KDmaHU<2> lb;
  lb.init([&](int q) { return reinterpret_cast<const char*>(q == 0 ? Wgq : Wuq) + wrow0 * d; },
          [&](int i) { return (uint32_t)(i & 63) * (uint32_t)d; });
  ScaleDmaH<2> sb;
  sb.init([&](int w) { return reinterpret_cast<const char*>(w == 0 ? sg : su) + wrow0 * 4; }, (int64_t)E * n * 4,
          [&](int i) { return (uint32_t)(i & 63) * 4u; });
  auto bsub = [&](int j) { return j * 64 + wn * 32; };
  AccW8 acc;
  gemm_mainloop_h_mx<FMT>(la, lb, sa, sb, d / 64, acc, L_0, L_1, L_2, wm, bsub);
  auto arow = [&](int r) { return (r < UP8H_ROWS ? L_0 + r * UP8H_ROW : L_1 + (r - UP8H_ROWS) * UP8H_ROW); };
  char* codes_lds = L_2;  // [256][MXC_ROW]
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    float a[16];
    float amax = 0.0f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float gv = acc.c[i][0][v], uv = acc.c[i][1][v];
      a[v] = (float)(bf16)(gv * sigmoid_f32(gv) * uv);  // the activation in the element type
      amax = fmaxf(amax, fabsf(a[v]));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    const int k = mx_exponent<FMT>(amax);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = wn * 32 + acc_n(4 * q);
      const int lo = mx_cvt2<FMT, false>(ldexpf(a[4 * q], -k), ldexpf(a[4 * q + 1], -k), 0);
      const int w = mx_cvt2<FMT, true>(ldexpf(a[4 * q + 2], -k), ldexpf(a[4 * q + 3], -k), lo);
      *reinterpret_cast<int*>(codes_lds + r * MXC_ROW + c) = w;
      if (act) {
        const u32x2 pk = {pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
        *reinterpret_cast<u32x2*>(arow(r) + c * 2) = pk;
      }
    }
    const int blk = (j0 >> 5) + wn;
    if (lane < 32 && r < g.mrows) sact[((int64_t)(blk >> 2) * R_max + g.m0 + r) * 4 + (blk & 3)] = (uint8_t)(k + 127);
  }
  __syncthreads();
  // codes: 256 rows x 64 bytes = 1024 chunks of 16 bytes, four per thread
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int c = threadIdx.x + b * GEMM_THREADS;
    const int r = c >> 2, ch = c & 3;
    const u32x4 v = *reinterpret_cast<const u32x4*>(codes_lds + r * MXC_ROW + ch * 16);
    if (r < g.mrows) st16_nt(act_q + (int64_t)(g.m0 + r) * n + j0 + ch * 16, v);
  }
  if (act) {
    bf16* out = act + (int64_t)g.m0 * n + j0;
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = threadIdx.x + b * GEMM_THREADS;
      const int r = c >> 3, ch = c & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(arow(r) + ch * 16);
      if (r < g.mrows) st16_nt(out + (int64_t)r * n + ch * 8, v);
    }
  }
}

// Down with block scales on the half-width engine: tile 256 rows x 128 columns of d.
template <int FMT>
__global__ __launch_bounds__(GEMM_THREADS, 2) void k_down_mx_h(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ sa_, const uint8_t* __restrict__ Wdq,
    const uint8_t* __restrict__ sd, bf16* __restrict__ Y, int d, int n, int E, int NT, int64_t R_max) {
  MOE_GEMM_LDS_HMX(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * HBN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // rows past the valid ones read the last valid row (never stored)
  const int vrows = min(HBN, d - n0);
  KDmaHU<4> la;
  la.init([&](int) { return reinterpret_cast<const char*>(Aq) + (int64_t)g.m0 * n; },
          [&](int i) { return (uint32_t)min(i, g.mrows - 1) * (uint32_t)n; });
  ScaleDmaH<4> sa;
  sa.init([&](int) { return reinterpret_cast<const char*>(sa_); }, R_max * 4,
          [&](int i) { return (uint32_t)(g.m0 + min(i, g.mrows - 1)) * 4u; });
  const int64_t wrow0 = (int64_t)g.e * d + n0;
  KDmaHU<2> lb;
  lb.init([&](int) { return reinterpret_cast<const char*>(Wdq) + wrow0 * n; },
          [&](int i) { return (uint32_t)min(i, vrows - 1) * (uint32_t)n; });
  ScaleDmaH<2> sb;
  sb.init([&](int) { return reinterpret_cast<const char*>(sd) + wrow0 * 4; }, (int64_t)E * d * 4,
          [&](int i) { return (uint32_t)min(i, vrows - 1) * 4u; });
  auto bsub = [&](int j) { return bsub_w8(wn, j); };
  AccW8 acc;
  gemm_mainloop_h_mx<FMT>(la, lb, sa, sb, n / 64, acc, L_0, L_1, L_2, wm, bsub);
  bf16* out = Y + (int64_t)g.m0 * d + n0;
  epi_h([&](int i, int j, int v) { return acc.c[i][j][v]; }, L_0, L_1, L_2, wm, bsub,
        [&](int r) { return out + (int64_t)r * d; }, g.mrows, vrows);
}

// Gate/up with block scales on the four-wave engine, for d > UP_H_MAX_D_FP8: tile 256 rows x 128
// act columns (B: W_gate rows j0 .. j0 + 127 over W_up rows j0 .. j0 + 127, halved block layout,
// so G and U of a (row, column) sit in accumulator blocks j and j + 2 of one lane).  Wave column
// wn holds act columns j0 + 64 wn .. + 63, two scale blocks (j = 0, 1), each split between lanes l
// and l + 32 as in k_up_mx_h.  Staging: the bf16 act in bytes 0-255 of each epilogue row, the codes
// in bytes 256-383.
template <int FMT>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_up_mx(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const int32_t* __restrict__ row_token, const uint8_t* __restrict__ Xq, const uint8_t* __restrict__ sx,
    const uint8_t* __restrict__ Wgq, const uint8_t* __restrict__ sg, const uint8_t* __restrict__ Wuq,
    const uint8_t* __restrict__ su, bf16* __restrict__ act, uint8_t* __restrict__ act_q,
    uint8_t* __restrict__ sact, int d, int n, int E, int NT, int64_t R_max, int T_) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int j0 = g.nt * 128;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int valid = min(128, n - j0);  // 64 or 128 (n is a multiple of 64)
  // rows and columns past the valid ones read the last valid one (never stored); gathered code
  // offsets fit in 32 bits (checked on the host: T * d < 2^32)
  auto rowi = [&](int i) { return g.m0 + min(i, g.mrows - 1); };
  KDmaHU<4> la;
  la.init([&](int) { return reinterpret_cast<const char*>(Xq); },
          [&](int i) { return (uint32_t)clamp_idx(row_token[rowi(i)], T_) * (uint32_t)d; });
  ScaleDmaH<4> sa;
  sa.init([&](int) { return reinterpret_cast<const char*>(sx); }, R_max * 4, [&](int i) { return (uint32_t)rowi(i) * 4u; });
  const int64_t wrow0 = (int64_t)g.e * n + j0;
  KDmaHU<4> lb;  // instructions 0, 1: W_gate rows; 2, 3: W_up rows
  lb.init([&](int q) { return reinterpret_cast<const char*>(q < 2 ? Wgq : Wuq) + wrow0 * d; },
          [&](int i) { return (uint32_t)min(i & 127, valid - 1) * (uint32_t)d; });
  ScaleDmaH<4> sb;  // waves 0, 1: W_gate rows; 2, 3: W_up rows
  sb.init([&](int w) { return reinterpret_cast<const char*>(w < 2 ? sg : su) + wrow0 * 4; }, (int64_t)E * n * 4,
          [&](int i) { return (uint32_t)min(i & 127, valid - 1) * 4u; });
  auto bsub = [&](int j) { return bsub_halved(wn, j); };
  WaveAcc acc;
  gemm_mainloop_f8_mx<FMT>(la, lb, sa, sb, d / 64, acc, L, wm, bsub);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = acc_m(wm, i);
    char* row = epi_row(L, r);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c0 = bsub(j);  // wn * 64 + 32 j
      float a[16];
      float amax = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float gv = acc.c[i][j][v], uv = acc.c[i][j + 2][v];
        a[v] = (float)(bf16)(gv * sigmoid_f32(gv) * uv);  // the activation in the element type
        amax = fmaxf(amax, fabsf(a[v]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int k = mx_exponent<FMT>(amax);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + acc_n(4 * q);
        const int lo = mx_cvt2<FMT, false>(ldexpf(a[4 * q], -k), ldexpf(a[4 * q + 1], -k), 0);
        const int w = mx_cvt2<FMT, true>(ldexpf(a[4 * q + 2], -k), ldexpf(a[4 * q + 3], -k), lo);
        *reinterpret_cast<int*>(row + 256 + c) = w;
        if (act) {
          const u32x2 pk = {pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
          *reinterpret_cast<u32x2*>(row + c * 2) = pk;
        }
      }
      const int blk = (j0 + c0) >> 5;
      if (lane < 32 && r < g.mrows && c0 < valid)
        sact[((int64_t)(blk >> 2) * R_max + g.m0 + r) * 4 + (blk & 3)] = (uint8_t)(k + 127);
    }
  }
  __syncthreads();
  // codes: 256 rows x 128 bytes = 2048 chunks of 16 bytes, eight per thread
  const int cvalid = valid / 16;
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int c = threadIdx.x + b * GEMM_THREADS;
    const int r = c >> 3, ch = c & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(epi_row(L, r) + 256 + ch * 16);
    if (r < g.mrows && ch < cvalid) st16_nt(act_q + (int64_t)(g.m0 + r) * n + j0 + ch * 16, v);
  }
  if (act) epi_store_bf16(L, 0, act + (int64_t)g.m0 * n + j0, n, g.mrows, 128, valid);
}

// Down with block scales on the four-wave engine, for n > DOWN_H_MAX_N_FP8: tile 256 rows x 256
// columns of d.
template <int FMT>
__global__ __launch_bounds__(GEMM_THREADS, 1) void k_down_mx(
    const int32_t* __restrict__ mtile_off, const int32_t* __restrict__ expert_off,
    const uint8_t* __restrict__ Aq, const uint8_t* __restrict__ sa_, const uint8_t* __restrict__ Wdq,
    const uint8_t* __restrict__ sd, bf16* __restrict__ Y, int d, int n, int E, int NT, int64_t R_max) {
  MOE_GEMM_LDS(L);
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  GroupTile g;
  if (!find_group_tile(lin, NT, mtile_off, expert_off, E, g)) return;
  const int n0 = g.nt * BN;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int vrows = min(BN, d - n0);
  KDmaHU<4> la;
  la.init([&](int) { return reinterpret_cast<const char*>(Aq) + (int64_t)g.m0 * n; },
          [&](int i) { return (uint32_t)min(i, g.mrows - 1) * (uint32_t)n; });
  ScaleDmaH<4> sa;
  sa.init([&](int) { return reinterpret_cast<const char*>(sa_); }, R_max * 4,
          [&](int i) { return (uint32_t)(g.m0 + min(i, g.mrows - 1)) * 4u; });
  const int64_t wrow0 = (int64_t)g.e * d + n0;
  KDmaHU<4> lb;
  lb.init([&](int) { return reinterpret_cast<const char*>(Wdq) + wrow0 * n; },
          [&](int i) { return (uint32_t)min(i, vrows - 1) * (uint32_t)n; });
  ScaleDmaH<4> sb;
  sb.init([&](int) { return reinterpret_cast<const char*>(sd) + wrow0 * 4; }, (int64_t)E * d * 4,
          [&](int i) { return (uint32_t)min(i, vrows - 1) * 4u; });
  auto bsub = [&](int j) { return bsub_plain(wn, j); };
  WaveAcc acc;
  gemm_mainloop_f8_mx<FMT>(la, lb, sa, sb, n / 64, acc, L, wm, bsub);
  epi_stage_bf16(L, wm, bsub, [&](int i, int j, int v) { return acc.c[i][j][v]; });
  __syncthreads();
  epi_store_bf16(L, 0, Y + (int64_t)g.m0 * d + n0, d, g.mrows, BN, vrows);
}

static inline int grid8f(int64_t n) { return (int)((n + 7) / 8 * 8); }

hipError_t launch_up_fp8(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, const uint8_t* Xq,
                         const float* sx, const uint8_t* Wgq, const float* sg, const uint8_t* Wuq,
                         const float* su, void* act, hipStream_t st) {
  if (s.d <= UP_H_MAX_D_FP8) {
    const int NT = (int)cdiv(s.n, UP8H_COLS);
    k_up_fp8_h<<<grid8f(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, p.row_token, Xq, sx, Wgq, sg, Wuq, su, static_cast<bf16*>(act), (int)s.d,
        (int)s.n, s.E, NT, (int)s.T);
  } else {
    const int NT = (int)cdiv(s.n, 128);
    k_up_fp8<<<grid8f(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, p.row_token, Xq, sx, Wgq, sg, Wuq, su, static_cast<bf16*>(act), (int)s.d,
        (int)s.n, s.E, NT, (int)s.T);
  }
  return hipGetLastError();
}

hipError_t launch_down_fp8(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, const uint8_t* Aq,
                           const float* sa, const uint8_t* Wdq, const float* sd, void* Y, hipStream_t st) {
  if (s.n <= DOWN_H_MAX_N_FP8) {
    const int NT = (int)cdiv(s.d, HBN);
    k_down_fp8_h<<<grid8f(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, Aq, sa, Wdq, sd, static_cast<bf16*>(Y), (int)s.d, (int)s.n, s.E, NT);
  } else {
    const int NT = (int)cdiv(s.d, BN);
    k_down_fp8<<<grid8f(max_mtiles(s.R_max, s.E) * NT), GEMM_THREADS, 0, st>>>(
        mtile_off, p.expert_off, Aq, sa, Wdq, sd, static_cast<bf16*>(Y), (int)s.d, (int)s.n, s.E, NT);
  }
  return hipGetLastError();
}

hipError_t launch_gather_mx_scales(const Shape& s, const PlanPtrs& p, const uint8_t* sx, uint8_t* sxp,
                                   hipStream_t st) {
  const int groups = (int)((s.d + 127) / 128);
  k_gather_mx_scales<<<(unsigned)((s.R_max + 255) / 256), 256, 0, st>>>(
      reinterpret_cast<const uint32_t*>(sx), p.row_token, p.meta, s.T, s.R_max, groups, reinterpret_cast<uint32_t*>(sxp));
  return hipGetLastError();
}

hipError_t launch_up_mx(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, int fmt, const uint8_t* Xq,
                        const uint8_t* sxp, const uint8_t* Wgq, const uint8_t* sg, const uint8_t* Wuq,
                        const uint8_t* su, void* act, uint8_t* act_q, uint8_t* sact, hipStream_t st) {
  const bool half = s.d <= UP_H_MAX_D_FP8;
  const int NT = (int)cdiv(s.n, half ? UP8H_COLS : 128);
  const int grid = grid8f(max_mtiles(s.R_max, s.E) * NT);
#define MOE_UPMX(K, F) K<F><<<grid, GEMM_THREADS, 0, st>>>(mtile_off, p.expert_off, p.row_token, Xq, sxp, Wgq, sg, \
      Wuq, su, static_cast<bf16*>(act), act_q, sact, (int)s.d, (int)s.n, s.E, NT, s.R_max, (int)s.T)
  if (half) { if (fmt == 0) MOE_UPMX(k_up_mx_h, 0); else MOE_UPMX(k_up_mx_h, 1); }
  else { if (fmt == 0) MOE_UPMX(k_up_mx, 0); else MOE_UPMX(k_up_mx, 1); }
#undef MOE_UPMX
  return hipGetLastError();
}

hipError_t launch_down_mx(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, int fmt, const uint8_t* Aq,
                          const uint8_t* sa, const uint8_t* Wdq, const uint8_t* sd, void* Y, hipStream_t st) {
  const bool half = s.n <= DOWN_H_MAX_N_FP8;
  const int NT = (int)cdiv(s.d, half ? HBN : BN);
  const int grid = grid8f(max_mtiles(s.R_max, s.E) * NT);
#define MOE_DNMX(K, F) K<F><<<grid, GEMM_THREADS, 0, st>>>(mtile_off, p.expert_off, Aq, sa, Wdq, sd, \
      static_cast<bf16*>(Y), (int)s.d, (int)s.n, s.E, NT, s.R_max)
  if (half) { if (fmt == 0) MOE_DNMX(k_down_mx_h, 0); else MOE_DNMX(k_down_mx_h, 1); }
  else { if (fmt == 0) MOE_DNMX(k_down_mx, 0); else MOE_DNMX(k_down_mx, 1); }
#undef MOE_DNMX
  return hipGetLastError();
}

}  // namespace moe

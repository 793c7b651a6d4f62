// Permute (materialised expert-major copy of the tokens) and the scatter-free weighted combine.
//
// Pages: cloud.baidu.com "工作原理" steps 2 and 4 (dispatch tokens to their experts, return the
// results to the tokens' positions; on one GPU both are local row movements); apxml.com
// "自定义核与核融合" step 5 (combine the expert outputs weighted by the gate scores); SonicMoE page
// kernel-comparison table (no separate scatter kernel: each token gathers its own rows, so no
// two workgroups ever write the same output row and no atomics are needed).
//
// Both kernels stream whole rows with 16-byte accesses, one 64-lane wave per token: the permute
// reads the token's row once and writes it to each of its expert-major rows (tok_row, the
// token-major inverse index; every destination row has exactly one source, so no atomics), the
// combine gathers the token's rows and accumulates them in fp32 in ascending expert order,
// rounding once.
#include "internal.h"

namespace moe {

// Lanes own 16-byte column chunks, PC per pass (a whole row of up to 64 * PC chunks is loaded
// once, then stored to every destination row).
template <typename T, int PC>
__global__ __launch_bounds__(256) void k_permute(const int32_t* __restrict__ tok_off,
                                                 const int32_t* __restrict__ tok_row,
                                                 const T* __restrict__ X, T* __restrict__ Xp, int d,
                                                 int T_, int rmax) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  const int base = tok_off[t], cnt = tok_off[t + 1] - base;
  constexpr int VEC = 16 / sizeof(T);
  const int nch = d / VEC;
  const T* s = X + (int64_t)t * d;
  for (int c0 = lane; c0 < nch; c0 += 64 * PC) {
    u32x4 v[PC];
#pragma unroll
    for (int q = 0; q < PC; ++q)
      if (c0 + 64 * q < nch) v[q] = ld16(s + (c0 + 64 * q) * VEC);
    for (int i = 0; i < cnt; ++i) {
      T* o = Xp + (int64_t)clamp_idx(tok_row[base + i], rmax) * d;
#pragma unroll
      for (int q = 0; q < PC; ++q)
        if (c0 + 64 * q < nch) st16_nt(o + (c0 + 64 * q) * VEC, v[q]);
    }
  }
}

hipError_t launch_permute(const Shape& s, const PlanPtrs& p, const void* X, void* X_perm, hipStream_t st) {
  const int grid = (int)cdiv(s.T, 4);
  const int rmax = (int)s.R_max;
  if (s.bf16)
    k_permute<bf16, 4><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, (const bf16*)X, (bf16*)X_perm, (int)s.d,
                                             (int)s.T, rmax);
  else
    k_permute<float, 4><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, (const float*)X, (float*)X_perm, (int)s.d,
                                              (int)s.T, rmax);
  return hipGetLastError();
}

// out[t] = sum_{r in rows(t)} w_r Y[r].  A wave owns a token; its lanes own CPL 16-byte column
// chunks each (lane + 64 j), so one pass covers 64 * CPL chunks of the row (the whole row when
// d is small enough; otherwise the row goes in several passes).  Per pass the rows are read in
// batches of RBATCH: every chunk of every row of a batch is requested before any is used, so a
// wave reads whole rows at once (RBATCH * CPL loads in flight per lane) instead of one chunk of
// each row per round trip.  fp32 accumulation in ascending expert order, one rounding.
template <typename T, bool WEIGHTED, int CPL, int RBATCH>
__global__ __launch_bounds__(256) void k_combine(const int32_t* __restrict__ tok_off,
                                                 const int32_t* __restrict__ tok_row,
                                                 const float* __restrict__ row_w,
                                                 const T* __restrict__ Y, T* __restrict__ out,
                                                 int T_, int d, int rmax) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T_) return;
  const int base = tok_off[t], cnt = tok_off[t + 1] - base;
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
    for (int i = 0; i < cnt; i += RBATCH) {
      u32x4 v[RBATCH][CPL];
      float w[RBATCH];
#pragma unroll
      for (int q = 0; q < RBATCH; ++q) {
        const bool live = i + q < cnt;
        const int r = live ? clamp_idx(tok_row[base + i + q], rmax) : 0;
        w[q] = live ? (WEIGHTED ? row_w[r] : 1.0f) : 0.0f;
        const T* y = Y + (int64_t)r * d + (int64_t)(c0 + lane) * VEC;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
          v[q][j] = (live && ok[j]) ? ld16_nt(y + 64 * j * VEC) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int q = 0; q < RBATCH; ++q) {
        if (i + q >= cnt) break;  // (uniform) the batch's rows past the token's last one add nothing
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          float f[VEC];
          unpack16<T>(v[q][j], f);
#pragma unroll
          for (int k = 0; k < VEC; ++k) acc[j][k] += w[q] * f[k];
        }
      }
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j)
      if (ok[j]) st16(out + (int64_t)t * d + (int64_t)(c0 + lane + 64 * j) * VEC, pack16<T>(acc[j]));
  }
}

template <typename T, bool W>
static void combine_for(const Shape& s, const PlanPtrs& p, const void* Y_perm, void* out, hipStream_t st) {
  const int grid = (int)cdiv(s.T, 4);
  const int64_t nch = s.d / (16 / (int)sizeof(T));
  const T* Y = static_cast<const T*>(Y_perm);
  T* o = static_cast<T*>(out);
  // chunks per lane: the whole row in one pass up to 4 * 64 chunks (bf16 d <= 2048), else passes
  // of 4 * 64 chunks; rows per batch keep RBATCH * CPL at 8 to 16 loads in flight per lane
  if (nch <= 64) k_combine<T, W, 1, 8><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, p.row_w, Y, o, (int)s.T, (int)s.d, (int)s.R_max);
  else if (nch <= 128) k_combine<T, W, 2, 8><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, p.row_w, Y, o, (int)s.T, (int)s.d, (int)s.R_max);
  else if (nch <= 192) k_combine<T, W, 3, 4><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, p.row_w, Y, o, (int)s.T, (int)s.d, (int)s.R_max);
  else k_combine<T, W, 4, 4><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, p.row_w, Y, o, (int)s.T, (int)s.d, (int)s.R_max);
}

hipError_t launch_combine(const Shape& s, const PlanPtrs& p, const void* Y_perm, bool weighted,
                          void* out, hipStream_t st) {
  if (s.bf16) { if (weighted) combine_for<bf16, true>(s, p, Y_perm, out, st); else combine_for<bf16, false>(s, p, Y_perm, out, st); }
  else { if (weighted) combine_for<float, true>(s, p, Y_perm, out, st); else combine_for<float, false>(s, p, Y_perm, out, st); }
  return hipGetLastError();
}

}  // namespace moe

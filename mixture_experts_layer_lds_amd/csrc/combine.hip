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

// out[t] = sum_{r in rows(t)} w_r Y[r].  Lanes own 16-byte column chunks; up to RB rows (a
// token's K = 8 rows at once in the common case) are loaded before they are accumulated so that
// several loads are in flight per lane.
constexpr int RB = 8;
template <typename T, bool WEIGHTED>
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
  for (int c = lane; c < nch; c += 64) {
    float acc[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) acc[k] = 0.0f;
    int i = 0;
    for (; i + RB <= cnt; i += RB) {
      u32x4 v[RB];
      float w[RB];
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        const int r = clamp_idx(tok_row[base + i + q], rmax);
        v[q] = ld16_nt(Y + (int64_t)r * d + c * VEC);
        w[q] = WEIGHTED ? row_w[r] : 1.0f;
      }
#pragma unroll
      for (int q = 0; q < RB; ++q) {
        float f[VEC];
        unpack16<T>(v[q], f);
#pragma unroll
        for (int k = 0; k < VEC; ++k) acc[k] += w[q] * f[k];
      }
    }
    for (; i < cnt; ++i) {
      const int r = clamp_idx(tok_row[base + i], rmax);
      const float w = WEIGHTED ? row_w[r] : 1.0f;
      float f[VEC];
      unpack16<T>(ld16_nt(Y + (int64_t)r * d + c * VEC), f);
#pragma unroll
      for (int k = 0; k < VEC; ++k) acc[k] += w * f[k];
    }
    st16(out + (int64_t)t * d + c * VEC, pack16<T>(acc));
  }
}

hipError_t launch_combine(const Shape& s, const PlanPtrs& p, const void* Y_perm, bool weighted,
                          void* out, hipStream_t st) {
  const int grid = (int)cdiv(s.T, 4);
#define MOE_COMB(TT, W) k_combine<TT, W><<<grid, 256, 0, st>>>(p.tok_off, p.tok_row, p.row_w, \
      (const TT*)Y_perm, (TT*)out, (int)s.T, (int)s.d, (int)s.R_max)
  if (s.bf16) { if (weighted) MOE_COMB(bf16, true); else MOE_COMB(bf16, false); }
  else { if (weighted) MOE_COMB(float, true); else MOE_COMB(float, false); }
#undef MOE_COMB
  return hipGetLastError();
}

}  // namespace moe

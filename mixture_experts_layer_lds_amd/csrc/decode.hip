// Single-launch MoE layer for small token counts (decode / inference).
//
// Pages: apxml.com "自定义核与核融合" (gate scores, top-k, gather of the selected experts'
// parameters, the experts' matmuls and the weighted combine fused into one kernel to avoid global
// round trips) and "条件参数加载" (only the selected experts' weights are read).
//
// At small T the layer is bound by reading the routed experts' weights, and launch count matters,
// so the whole forward is one cooperative kernel whose workgroups pass five phases separated by
// grid-wide barriers (every workgroup walks every phase with grid-stride loops, so each reaches
// every barrier):
//   A. router logits (+ bias) and top-K with softmax, one token per workgroup;
//   B. per-expert token lists, in ascending (token, k) order;
//   C. gate/up: each unit is 32 rows of [W_gate; W_up][e] for one expert with tokens; every
//      weight row is streamed once (8 lanes x 16 bytes per 128-byte line) and dotted with all of
//      the expert's tokens (x staged in LDS) -> h[pair][2n] in fp32;
//   D. SwiGLU + down: each unit is 32 rows (output columns) of W_down[e]; act = silu(G) U is
//      built from h into LDS, dotted with every row -> y[pair][d] in fp32;
//   E. combine: out[t] = sum over the token's experts, in ascending expert order, of w y.
// Routing is plain top-K (no token rounding); results match moe_forward up to rounding (the
// activation is kept in fp32 here instead of being rounded to the element type).
#include "internal.h"

#include <hip/hip_cooperative_groups.h>

namespace moe {

namespace cg = cooperative_groups;

constexpr int DEC_THREADS = 256;
constexpr int DEC_ROWS = 32;     // weight rows per unit (8 lanes per row)
constexpr int DEC_TOK = 16;      // tokens per pass over a unit's rows
constexpr int DEC_DBLK = 512;    // reduction elements staged in LDS per block

struct DecodeArgs {
  const void* X;
  const void* W_r;
  const float* bias;
  const void* W_gate;
  const void* W_up;
  const void* W_down;
  float* logits;
  int32_t* topk_idx;
  float* topk_w;
  void* out;
  int32_t* cnt;   // [E]
  int32_t* list;  // [E][T] pair ids t * K + k
  float* h;       // [T * K][2n]
  float* y;       // [T * K][d]
  int T, d, n, E, K;
};

__device__ __forceinline__ uint32_t dec_order_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename T>
__device__ __forceinline__ float dot8(u32x4 w, const float* x) {
  float f[8];
  if constexpr (sizeof(T) == 2) {
    unpack16<bf16>(w, f);
  } else {
    unpack16<float>(w, f);  // 4 elements; the caller passes 4-element chunks for fp32
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < (int)(16 / sizeof(T)); ++i) s += f[i] * x[i];
  return s;
}

// One unit of phase C or D: rows row0 .. row0 + 31 of a weight matrix whose row r starts at
// wrow(r) (K_len elements), dotted with the vectors of up to DEC_TOK tokens held in LDS as fp32
// (xs[tok][DEC_DBLK], refilled block by block by fill(tok, k0, k1)).  Returns through emit(tok,
// row, value) on the lane that owns the row's sum (sub-lane 0 of each 8-lane group).
template <typename T, class WRow, class Fill, class Emit>
__device__ void dec_unit(int nrows, int row0, int K_len, int ntok, WRow wrow, Fill fill, Emit emit,
                         float* xs) {
  constexpr int VEC = 16 / sizeof(T);
  const int tid = threadIdx.x;
  const int r = tid >> 3, part = tid & 7;  // row within the unit, lane within the row's group
  const int row = row0 + r;
  const bool live = row < nrows;
  const T* wr = live ? reinterpret_cast<const T*>(wrow(row)) : nullptr;
  float acc[DEC_TOK];
#pragma unroll
  for (int i = 0; i < DEC_TOK; ++i) acc[i] = 0.0f;
  for (int k0 = 0; k0 < K_len; k0 += DEC_DBLK) {
    const int k1 = min(K_len, k0 + DEC_DBLK);
    __syncthreads();
    fill(ntok, k0, k1);
    __syncthreads();
    if (live) {
      for (int k = k0 + part * VEC; k < k1; k += 8 * VEC) {
        const u32x4 w = ld16(wr + k);
#pragma unroll
        for (int i = 0; i < DEC_TOK; ++i)
          if (i < ntok) acc[i] += dot8<T>(w, xs + i * DEC_DBLK + (k - k0));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < DEC_TOK; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 1, 64);
    v += __shfl_xor(v, 2, 64);
    v += __shfl_xor(v, 4, 64);
    if (live && part == 0 && i < ntok) emit(i, row, v);
  }
}

template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_decode(DecodeArgs a) {
  cg::grid_group grid = cg::this_grid();
  extern __shared__ float dsm[];  // [DEC_TOK][DEC_DBLK] fp32 staging, reused by every phase
  __shared__ float s_log[1024];
  constexpr int VEC = 16 / sizeof(T);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* X = reinterpret_cast<const T*>(a.X);
  const int T_ = a.T, d = a.d, n = a.n, E = a.E, K = a.K;

  // ---- A: router + top-K, one token per workgroup ----
  for (int t = blockIdx.x; t < T_; t += gridDim.x) {
    const T* xt = X + (int64_t)t * d;
    const T* Wr = reinterpret_cast<const T*>(a.W_r);
    for (int e = wave; e < E; e += DEC_THREADS / 64) {
      float s = 0.0f;
      for (int c = lane * VEC; c < d; c += 64 * VEC) {
        float xf[8], wf[8];
        unpack16<T>(ld16(xt + c), xf);
        unpack16<T>(ld16(Wr + (int64_t)e * d + c), wf);
#pragma unroll
        for (int i = 0; i < VEC; ++i) s += xf[i] * wf[i];
      }
      s = wave_sum(s);
      if (lane == 0) {
        const float L = s + (a.bias ? a.bias[e] : 0.0f);
        s_log[e] = L;
        a.logits[(int64_t)t * E + e] = L;
      }
    }
    __syncthreads();
    if (wave == 0) {
      // composite keys (order_key(L) << 32) | ~e: one unsigned maximum orders by logit
      // descending, then expert id ascending; lane i holds experts i + 64 j (E <= 1024)
      uint64_t ck[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        ck[j] = e < E ? (((uint64_t)dec_order_key(s_log[e]) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
      }
      int my_e = 0;
      for (int k = 0; k < K; ++k) {
        uint64_t b = 0ull;
#pragma unroll
        for (int j = 0; j < 16; ++j) b = ck[j] > b ? ck[j] : b;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint64_t x = __shfl_xor(b, o, 64);
          b = x > b ? x : b;
        }
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (ck[j] == b) ck[j] = 0ull;
        const int win = (int)~(uint32_t)b;
        if (lane == 0) a.topk_idx[(int64_t)t * K + k] = win;
        if (lane == k) my_e = win;
      }
      const float my_v = lane < K ? s_log[my_e] : 0.0f;
      const float vmax = __shfl(my_v, 0, 64);
      const float ex = lane < K ? __expf(my_v - vmax) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < K) a.topk_w[(int64_t)t * K + lane] = ex / sum;
    }
    __syncthreads();
  }
  grid.sync();

  // ---- B: per-expert token lists in ascending (t, k) order ----
  {
    __shared__ int s_wcnt[DEC_THREADS / 64];
    const int P = T_ * K;
    for (int e = blockIdx.x; e < E; e += gridDim.x) {
      int base = 0;
      for (int p0 = 0; p0 < P; p0 += DEC_THREADS) {
        const int p = p0 + tid;
        const bool hit = p < P && a.topk_idx[p] == e;
        const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
        if (lane == 0) s_wcnt[wave] = (int)__builtin_popcountll(m);
        __syncthreads();
        int off = base;
        for (int w = 0; w < wave; ++w) off += s_wcnt[w];
        if (hit) a.list[(int64_t)e * T_ + off + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = p;
        int tot = 0;
        for (int w = 0; w < DEC_THREADS / 64; ++w) tot += s_wcnt[w];
        base += tot;
        __syncthreads();
      }
      if (tid == 0) a.cnt[e] = base;
    }
  }
  grid.sync();

  // ---- C: gate/up rows dotted with each routed token's x ----
  {
    const int nb = (2 * n + DEC_ROWS - 1) / DEC_ROWS;
    const T* Wg = reinterpret_cast<const T*>(a.W_gate);
    const T* Wu = reinterpret_cast<const T*>(a.W_up);
    for (int u = blockIdx.x; u < E * nb; u += gridDim.x) {
      const int e = u / nb, rb = u % nb;
      const int c = a.cnt[e];
      for (int g0 = 0; g0 < c; g0 += DEC_TOK) {
        const int ntok = min(DEC_TOK, c - g0);
        const int32_t* lst = a.list + (int64_t)e * T_ + g0;
        auto wrow = [&](int j) -> const void* {
          return j < n ? Wg + ((int64_t)e * n + j) * d : Wu + ((int64_t)e * n + (j - n)) * d;
        };
        auto fill = [&](int nt, int k0, int k1) {
          for (int i = tid; i < nt * DEC_DBLK; i += DEC_THREADS) {
            const int tk = i / DEC_DBLK, k = k0 + i % DEC_DBLK;
            const int t = lst[tk] / K;
            dsm[i] = k < k1 ? to_f32(X[(int64_t)t * d + k]) : 0.0f;
          }
        };
        auto emit = [&](int tk, int j, float v) { a.h[(int64_t)lst[tk] * 2 * n + j] = v; };
        dec_unit<T>(2 * n, rb * DEC_ROWS, d, ntok, wrow, fill, emit, dsm);
      }
    }
  }
  grid.sync();

  // ---- D: act = silu(G) U, dotted with W_down rows ----
  {
    const int nb = (d + DEC_ROWS - 1) / DEC_ROWS;
    const T* Wd = reinterpret_cast<const T*>(a.W_down);
    for (int u = blockIdx.x; u < E * nb; u += gridDim.x) {
      const int e = u / nb, cb = u % nb;
      const int c = a.cnt[e];
      for (int g0 = 0; g0 < c; g0 += DEC_TOK) {
        const int ntok = min(DEC_TOK, c - g0);
        const int32_t* lst = a.list + (int64_t)e * T_ + g0;
        auto wrow = [&](int col) -> const void* { return Wd + ((int64_t)e * d + col) * n; };
        auto fill = [&](int nt, int k0, int k1) {
          for (int i = tid; i < nt * DEC_DBLK; i += DEC_THREADS) {
            const int tk = i / DEC_DBLK, j = k0 + i % DEC_DBLK;
            float v = 0.0f;
            if (j < k1) {
              const float* hp = a.h + (int64_t)lst[tk] * 2 * n;
              const float G = hp[j], U = hp[n + j];
              v = G * sigmoid_f32(G) * U;
            }
            dsm[i] = v;
          }
        };
        auto emit = [&](int tk, int col, float v) { a.y[(int64_t)lst[tk] * d + col] = v; };
        dec_unit<T>(d, cb * DEC_ROWS, n, ntok, wrow, fill, emit, dsm);
      }
    }
  }
  grid.sync();

  // ---- E: combine in ascending expert order ----
  for (int t = blockIdx.x; t < T_; t += gridDim.x) {
    int ord[16];
    for (int k = 0; k < K; ++k) ord[k] = k;
    for (int k = 1; k < K; ++k) {  // insertion sort of the token's k by expert id (K <= 16)
      const int x = ord[k];
      int j = k - 1;
      while (j >= 0 && a.topk_idx[(int64_t)t * K + ord[j]] > a.topk_idx[(int64_t)t * K + x]) {
        ord[j + 1] = ord[j];
        --j;
      }
      ord[j + 1] = x;
    }
    T* out = reinterpret_cast<T*>(a.out) + (int64_t)t * d;
    for (int col = tid; col < d; col += DEC_THREADS) {
      float s = 0.0f;
      for (int q = 0; q < K; ++q) {
        const int k = ord[q];
        s += a.topk_w[(int64_t)t * K + k] * a.y[((int64_t)t * K + k) * d + col];
      }
      out[col] = from_f32<T>(s);
    }
  }
}

size_t decode_workspace_bytes(int64_t T, int64_t d, int64_t n, int E, int K) {
  const size_t a = ((size_t)E * 4 + 255) / 256 * 256;
  const size_t b = ((size_t)E * T * 4 + 255) / 256 * 256;
  const size_t c = ((size_t)T * K * 2 * n * 4 + 255) / 256 * 256;
  const size_t y = ((size_t)T * K * d * 4 + 255) / 256 * 256;
  return a + b + c + y;
}

hipError_t launch_decode(const Shape& s, const void* X, const void* W_r, const float* bias,
                         const void* W_gate, const void* W_up, const void* W_down, float* logits,
                         int32_t* topk_idx, float* topk_w, void* out, void* ws, hipStream_t st) {
  DecodeArgs a;
  a.X = X; a.W_r = W_r; a.bias = bias; a.W_gate = W_gate; a.W_up = W_up; a.W_down = W_down;
  a.logits = logits; a.topk_idx = topk_idx; a.topk_w = topk_w; a.out = out;
  char* w = static_cast<char*>(ws);
  a.cnt = reinterpret_cast<int32_t*>(w);
  w += ((size_t)s.E * 4 + 255) / 256 * 256;
  a.list = reinterpret_cast<int32_t*>(w);
  w += ((size_t)s.E * s.T * 4 + 255) / 256 * 256;
  a.h = reinterpret_cast<float*>(w);
  w += ((size_t)s.T * s.K * 2 * s.n * 4 + 255) / 256 * 256;
  a.y = reinterpret_cast<float*>(w);
  a.T = (int)s.T; a.d = (int)s.d; a.n = (int)s.n; a.E = s.E; a.K = s.K;
  const void* fn = s.bf16 ? reinterpret_cast<const void*>(&k_decode<bf16>)
                          : reinterpret_cast<const void*>(&k_decode<float>);
  const size_t lds = (size_t)DEC_TOK * DEC_DBLK * sizeof(float);
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, DEC_THREADS, lds);
  if (e != hipSuccess) return e;
  if (per_cu < 1) return hipErrorInvalidConfiguration;
  // every workgroup must be resident at once for the grid barriers: the cooperative launch
  // refuses a larger grid
  const int grid = cus * per_cu;
  void* params[] = {&a};
  return hipLaunchCooperativeKernel(fn, dim3(grid), dim3(DEC_THREADS), params, (unsigned)lds, st);
}

}  // namespace moe

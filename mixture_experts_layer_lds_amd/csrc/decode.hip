// Single-launch MoE layer for small token counts (decode / inference).
//
// Pages: apxml.com "自定义核与核融合" (gate scores, top-k, gather of the selected experts'
// parameters, the experts' matmuls and the weighted combine fused into one kernel to avoid global
// round trips) and "条件参数加载" (only the selected experts' weights are read).
//
// At small T every routed expert sees only a handful of tokens, so each projection is a skinny
// product [rows x k] x [k x tokens] bound by reading the expert's weights once.  Each such
// product runs on MFMA (16x16 tiles: 16 weight rows by 16 tokens), with the weight rows streamed
// straight from HBM into the A operand, several 16-byte loads in flight per lane, and the token
// vectors loaded into the B operand from L2.
//
// A tile is taken by a group of W waves of one workgroup (W = 1, 2, 4, 8 or 16, chosen per phase
// from the tile count and the reduction length to balance the grid): the members split the
// reduction, and member 0 adds their partial tiles from LDS in member order and runs the
// epilogue.  Members hand over through LDS counters (two buffers per group, so members run at
// most one tile ahead), never through a workgroup barrier; with W = 1 the wave does the whole
// tile alone.  Every result is deterministic.
//
// One kernel, one workgroup of 16 waves per CU (the whole grid resident at once), phases
// separated by grid-wide barriers (every workgroup walks every phase with grid-stride loops, so
// each reaches every barrier).  The barrier is a release fence, one relaxed arrival on a 64-bit counter, relaxed
// polling and an acquire fence: cache maintenance happens once per workgroup and barrier, not
// once per poll.  The counter lives in the call's workspace and a one-workgroup kernel clears it
// (with the per-expert counters) right before the launch, so calls share no device state and
// need no ordering beyond their workspace's stream.  A workgroup that polls longer than the spin
// limit (about a second) gives up: it raises the device's status word and leaves the kernel, so
// the workgroups still waiting give up at the next barrier and every one of them exits;
// moe_decode_status() reports and clears the word.  Phases:
//   A. router logits (+ bias): tiles of 16 experts x 16 tokens;
//   B. per token (one wave): top-K with softmax, and the token's (t, k) pairs appended to the
//      chosen experts' lists (the order inside a list does not affect any value: each token is
//      its own MFMA column);
//   C. gate/up: a tile holds 8 gate rows and the 8 matching up rows of one routed expert, so
//      the epilogue has G and U of the same column in lanes l and l + 32 and writes
//      act = silu(G) U in the element type (as the grouped forward does);
//   D. down: 16 rows of W_down[e] (output columns) against act -> y[pair][d] in fp32;
//   E. combine: out[t] = sum over the token's experts, in ascending expert order, of w y.
// Routing is plain top-K (no token rounding); results match moe_forward up to the order of the
// fp32 accumulations.
#include <atomic>

#include "internal.h"

namespace moe {

constexpr int DEC_THREADS = 1024;  // 16 waves per workgroup, one workgroup per CU
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_U = 4;           // reduction steps per batch with one token group (two batches in flight)
constexpr int DEC_NG = 3;          // token groups of 16 per pass over a tile's weight rows

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
  unsigned long long* bar;  // grid-barrier arrivals (cleared before the launch)
  int32_t* cnt;             // [E] (cleared before the launch)
  int32_t* list;            // [E][T] pair ids t * K + k
  void* act;                // [T * K][n] element type
  float* y;                 // [T * K][d]
  int T, d, n, E, K;
  long long spin_limit;     // polls before a grid barrier gives up
};

// One reduction step of a 16x16 tile: every lane holds 16 bytes of its weight row (A, row
// lane % 16) and 16 bytes of its token's vector (B, column lane % 16), both at the same k offset
// (lane / 16) * V inside the step, so the products pair the same k on both sides.
template <typename T> struct DecMma;
template <> struct DecMma<bf16> {
  static constexpr int S = 32;  // k elements per step
  static constexpr int V = 8;   // k elements per lane per step
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct DecMma<float> {
  static constexpr int S = 16;
  static constexpr int V = 4;
  __device__ static f32x4 mma(u32x4 a, u32x4 b, f32x4 c) {
    // four k = 4 products; product i takes element i of every lane's 4-element chunk
#pragma unroll
    for (int i = 0; i < 4; ++i)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), c, 0, 0, 0);
    return c;
  }
};

// Steps per batch: the register budget holds two batches of (1 + NG) 16-byte operands.
template <int NG> struct DecBatch { static constexpr int U = NG <= 2 ? DEC_U : DEC_U / 2; };

template <typename T, int NG>
struct DecStream {
  static constexpr int U = DecBatch<NG>::U;
  const T* w;       // lane's weight row at its k offset
  const T* x[NG];   // lane's token vectors at its k offset

  // steps st .. st + U - 1, constant offsets from one base per operand
  __device__ __forceinline__ void load(u32x4 (&wv)[U], u32x4 (&xv)[NG][U], int st) const {
    constexpr int S = DecMma<T>::S;
    const T* wp = w + st * S;
    const T* xp[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) xp[g] = x[g] + st * S;
#pragma unroll
    for (int u = 0; u < U; ++u) {  // in the order the MFMAs consume them
      wv[u] = ld16(wp + u * S);
#pragma unroll
      for (int g = 0; g < NG; ++g) xv[g][u] = ld16(xp[g] + u * S);
    }
  }
};

template <typename T, int NG, int U>
__device__ __forceinline__ void dec_mma(const u32x4 (&wv)[U], const u32x4 (&xv)[NG][U], f32x4 (&acc)[NG]) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = DecMma<T>::mma(wv[u], xv[g][u], acc[g]);
  }
}

// Steps [a, b) of one wave (a, b wave-uniform): whole batches with two register sets, the next
// batch's loads issued before the MFMAs of the current one, then the last (b - a) mod U steps
// as one short batch.
template <typename T, int NG>
__device__ __forceinline__ void dec_stream(const DecStream<T, NG>& ds, int a, int b, f32x4* acc) {
  constexpr int U = DecBatch<NG>::U;
  constexpr int S = DecMma<T>::S;
  f32x4 (&ac)[NG] = *reinterpret_cast<f32x4(*)[NG]>(acc);
  const int nfull = (b - a) / U;
  if (nfull > 0) {
    u32x4 w0[U], x0[NG][U], w1[U], x1[NG][U];
    ds.load(w0, x0, a);
    int i = 0;
    for (; i + 2 < nfull; i += 2) {  // steady state: loads unconditional, so the waits stay partial
      ds.load(w1, x1, a + (i + 1) * U);
      dec_mma<T, NG, U>(w0, x0, ac);
      ds.load(w0, x0, a + (i + 2) * U);
      dec_mma<T, NG, U>(w1, x1, ac);
    }
    if (i + 1 < nfull) {
      ds.load(w1, x1, a + (i + 1) * U);
      dec_mma<T, NG, U>(w0, x0, ac);
      dec_mma<T, NG, U>(w1, x1, ac);
    } else {
      dec_mma<T, NG, U>(w0, x0, ac);
    }
  }
  const int st = a + nfull * U, r = b - st;
  if (r > 0) {  // one more batch, all of its loads in flight together; steps past b repeat b - 1
    u32x4 wt[U], xt[NG][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int su = st + min(u, r - 1);
      wt[u] = ld16(ds.w + su * S);
#pragma unroll
      for (int g = 0; g < NG; ++g) xt[g][u] = ld16(ds.x[g] + su * S);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < r) {
#pragma unroll
        for (int g = 0; g < NG; ++g) ac[g] = DecMma<T>::mma(wt[u], xt[g][u], ac[g]);
      }
    }
  }
}

// Per-workgroup LDS: partial tiles [wave][buffer][token group][lane] and, per group, the
// arrival and consumption counters of its two buffers.
struct DecLds {
  f32x4 part[DEC_WAVES * 2 * DEC_NG * 64];
  int arrive[DEC_WAVES][2];
  int consumed[DEC_WAVES][2];
  int active[1024];  // routed experts in ascending order
  int nactive;
  int proceed;       // set by the barrier: 0 if this workgroup gave up waiting
};

__device__ __forceinline__ void dec_lds_wait_ge(int* p, int target) {
  // members of a group are waves of one resident workgroup: every wait ends
  while (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target)
    __builtin_amdgcn_s_sleep(1);
}

// One wave's view of the tile groups of a phase: W waves per group, this wave is member m of
// group grp (grid-wide index gid among ngroups groups), seq counts the group's tiles so far.
struct DecGroup {
  int W, m, grp, gid, ngroups, seq;
  __device__ __forceinline__ void setup(int w) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    W = w;
    m = wave % w;
    grp = wave / w;
    gid = blockIdx.x * (DEC_WAVES / w) + grp;
    ngroups = gridDim.x * (DEC_WAVES / w);
    seq = 0;
  }
};

// Wave count per tile for a phase with `items` tiles of `ns` reduction steps: the W in
// {1, 2, 4, 8, 16} that minimises rounds x (steps per member + a fixed cost per tile, about
// eight steps' worth for the first load's latency and the hand-over), where rounds =
// ceil(items W / waves in the grid); ties go to the smaller W.
__device__ __forceinline__ int dec_pick_w(int items, int ns) {
  const int waves = (int)gridDim.x * DEC_WAVES;
  int best_w = 1, best = 0x7fffffff;
  for (int w = 1; w <= DEC_WAVES; w *= 2) {
    if (w > 1 && ns < w) break;
    const int rounds = (items * w + waves - 1) / waves;
    const int cost = rounds * ((ns + w - 1) / w + 8);
    if (cost < best) {
      best = cost;
      best_w = w;
    }
  }
  return best_w;
}

// The group's tile: member m streams its share of steps [s0, s1) for ng token groups; the
// epilogue epi(v) runs on member 0 with the tile summed over members (v[g], rows 4 (lane / 16)
// + i, column lane % 16 of token group g).
template <typename T, class Epi>
__device__ __forceinline__ void dec_group_tile(DecGroup& G, DecLds& L, const T* wrow, const T* const* xrow,
                                               int ng, int s0, int s1, Epi epi) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ko = (lane >> 4) * DecMma<T>::V;
  const int ns = s1 - s0;
  const int a = s0 + ns * G.m / G.W, b = s0 + ns * (G.m + 1) / G.W;
  f32x4 acc[DEC_NG];
#pragma unroll
  for (int g = 0; g < DEC_NG; ++g) acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (ng == 3) {
    DecStream<T, 3> ds;
    ds.w = wrow + ko;
#pragma unroll
    for (int g = 0; g < 3; ++g) ds.x[g] = xrow[g] + ko;
    dec_stream<T, 3>(ds, a, b, acc);
  } else if (ng == 2) {
    DecStream<T, 2> ds;
    ds.w = wrow + ko;
    ds.x[0] = xrow[0] + ko;
    ds.x[1] = xrow[1] + ko;
    dec_stream<T, 2>(ds, a, b, acc);
  } else {
    DecStream<T, 1> ds;
    ds.w = wrow + ko;
    ds.x[0] = xrow[0] + ko;
    dec_stream<T, 1>(ds, a, b, acc);
  }
  if (G.W == 1) {
    epi(acc);
    return;
  }
  const int buf = G.seq & 1, use = G.seq >> 1;
  ++G.seq;
  dec_lds_wait_ge(&L.consumed[G.grp][buf], use);  // the buffer's previous tile has been read
  for (int g = 0; g < ng; ++g) L.part[((wave * 2 + buf) * DEC_NG + g) * 64 + lane] = acc[g];
  if (lane == 0) __hip_atomic_fetch_add(&L.arrive[G.grp][buf], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (G.m == 0) {
    dec_lds_wait_ge(&L.arrive[G.grp][buf], (use + 1) * G.W);
    f32x4 v[DEC_NG];
    for (int g = 0; g < ng; ++g) {
      v[g] = L.part[((wave * 2 + buf) * DEC_NG + g) * 64 + lane];
      for (int mm = 1; mm < G.W; ++mm) v[g] += L.part[(((wave + mm) * 2 + buf) * DEC_NG + g) * 64 + lane];
    }
    if (lane == 0) __hip_atomic_store(&L.consumed[G.grp][buf], use + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    epi(v);
  }
}

__device__ __forceinline__ uint32_t dec_order_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float dec_key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

template <typename T>
__device__ __forceinline__ void dec_store4(T* p, f32x4 v) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[0])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[1])) << 16);
    const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[2])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<bf16>(v[3])) << 16);
    *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}

// Experts with at least one routed token, in ascending order, built by wave 0 of every
// workgroup into its LDS (list[i] = the i-th active expert); returns their number.
__device__ __forceinline__ int dec_active_experts(const int32_t* cnt, int E, int* list, int* count) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < 64) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const bool on = e < E && cnt[e] > 0;
      const uint64_t m = __builtin_amdgcn_ballot_w64(on);
      if (on) list[base + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = e;
      base += (int)__builtin_popcountll(m);
    }
    if (lane == 0) *count = base;
  }
  __syncthreads();
  return *count;
}

// Set when a workgroup gave up waiting at a grid barrier; read and cleared by
// moe_decode_status() (one word per device: each device holds its own copy).
__device__ int g_dec_status;

// Grid-wide barrier on the call's arrival counter, which only grows from zero: with nb
// workgroups, arrival number v belongs to the barrier that completes when the counter reaches
// (v / nb + 1) nb.  Also clears the workgroup's tile-group counters for the next phase.
// Returns false if this workgroup gave up (the status word is then set): the caller leaves the
// kernel, whose later phases would read results that were never written.
__device__ __forceinline__ bool dec_grid_barrier(unsigned long long* ctr, long long spin_limit, DecLds& L) {
  __builtin_amdgcn_s_waitcnt(0);  // this wave's loads and stores have completed
  __syncthreads();
  if (threadIdx.x < DEC_WAVES * 2) {
    (&L.arrive[0][0])[threadIdx.x] = 0;
    (&L.consumed[0][0])[threadIdx.x] = 0;
  }
  if (threadIdx.x == 0) {
    const unsigned long long nb = gridDim.x;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const unsigned long long v = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long target = (v / nb + 1) * nb;
    // bounded wait: with the grid resident every workgroup arrives, so the limit is only reached
    // if part of the grid could not be placed (other work holding CUs past the bound); then the
    // call reports an error instead of hanging or finishing with wrong results
    int ok = 0;
    for (long long spin = 0; spin < spin_limit; ++spin) {
      if (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= target) {
        ok = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) __hip_atomic_store(&g_dec_status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    L.proceed = ok;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  return L.proceed != 0;
}

// Clears a call's barrier counter and per-expert token counters before the decode kernel.
__global__ __launch_bounds__(256) void k_dec_clear(unsigned long long* bar, int32_t* cnt, int E) {
  if (threadIdx.x == 0) *bar = 0ull;
  for (int i = threadIdx.x; i < E; i += 256) cnt[i] = 0;
}

template <typename T>
__global__ __launch_bounds__(DEC_THREADS) void k_decode(DecodeArgs a) {
  unsigned long long* bar = a.bar;
  __shared__ DecLds L;
  constexpr int S = DecMma<T>::S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r16 = lane & 15, q = lane >> 4;
  const T* X = reinterpret_cast<const T*>(a.X);
  const int T_ = a.T, d = a.d, n = a.n, E = a.E, K = a.K;
  if (tid < DEC_WAVES * 2) {
    (&L.arrive[0][0])[tid] = 0;
    (&L.consumed[0][0])[tid] = 0;
  }
  __syncthreads();
  DecGroup G;

  // ---- A: router logits ----
  {
    const T* Wr = reinterpret_cast<const T*>(a.W_r);
    const int tiles = (E + 15) / 16, groups = (T_ + 15) / 16, passes = (groups + DEC_NG - 1) / DEC_NG;
    const int items = tiles * passes;
    G.setup(dec_pick_w(items, d / S));
    for (int u = G.gid; u < items; u += G.ngroups) {
      const int pass = u % passes, tile = u / passes;
      const T* wrow = Wr + (int64_t)min(tile * 16 + r16, E - 1) * d;
      const int g0 = pass * DEC_NG, ng = min(DEC_NG, groups - g0);
      const T* xr[DEC_NG];
#pragma unroll
      for (int g = 0; g < DEC_NG; ++g) xr[g] = X + (int64_t)min((g0 + g) * 16 + r16, T_ - 1) * d;
      dec_group_tile<T>(G, L, wrow, xr, ng, 0, d / S, [&](const f32x4* v) {
        for (int g = 0; g < ng; ++g) {
          const int t = (g0 + g) * 16 + r16;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = tile * 16 + 4 * q + i;
            if (t < T_ && e < E) a.logits[(int64_t)t * E + e] = v[g][i] + (a.bias ? a.bias[e] : 0.0f);
          }
        }
      });
    }
  }
  if (!dec_grid_barrier(bar, a.spin_limit, L)) return;

  // ---- B: top-K + softmax, per-expert lists; one token per wave ----
  {
    const int nw = gridDim.x * DEC_WAVES;
    for (int t = blockIdx.x * DEC_WAVES + wave; t < T_; t += nw) {
      // lane i holds the order keys of experts i + 64 j (E <= 1024); each round takes the largest
      // key still in play (a DPP wave maximum) and, among the experts holding it, the lowest id
      // (ballots in ascending e): logit descending, then expert id ascending
      const int ej = (E + 63) >> 6;
      uint32_t key[16];
      uint32_t alive = 0;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int e = lane + 64 * j;
        key[j] = e < E ? dec_order_key(a.logits[(int64_t)t * E + e]) : 0u;
        alive |= e < E ? (1u << j) : 0u;
      }
      int my_e = 0;
      float my_v = 0.0f;
      for (int k = 0; k < K; ++k) {
        uint32_t lm = 0;  // NaN keys are 0 too; ties at 0 are settled among live candidates
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if (j < ej && ((alive >> j) & 1u)) lm = key[j] > lm ? key[j] : lm;
        const uint32_t kmax = wave_max_u32(lm);
        int win = -1;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if (j >= ej) break;
          const uint64_t m = __builtin_amdgcn_ballot_w64(((alive >> j) & 1u) && key[j] == kmax);
          if (win < 0 && m != 0ull) win = 64 * j + (int)__builtin_ctzll(m);
        }
        win = __builtin_amdgcn_readfirstlane(win);
        if (lane == (win & 63)) alive &= ~(1u << (win >> 6));
        if (lane == k) {
          my_e = win;
          my_v = dec_key_value(kmax);
        }
      }
      const float vmax = __shfl(my_v, 0, 64);
      const float ex = lane < K ? __expf(my_v - vmax) : 0.0f;
      const float sum = wave_sum(ex);
      if (lane < K) {
        a.topk_idx[(int64_t)t * K + lane] = my_e;
        a.topk_w[(int64_t)t * K + lane] = ex / sum;
        const int pos = atomicAdd(&a.cnt[my_e], 1);  // < T: a token picks an expert at most once
        a.list[(int64_t)my_e * T_ + pos] = t * K + lane;
      }
    }
  }
  if (!dec_grid_barrier(bar, a.spin_limit, L)) return;

  const int nact = dec_active_experts(a.cnt, E, L.active, &L.nactive);

  // ---- C: gate/up tiles (8 gate + 8 up rows) -> act = silu(G) U ----
  {
    const T* Wg = reinterpret_cast<const T*>(a.W_gate);
    const T* Wu = reinterpret_cast<const T*>(a.W_up);
    T* act = reinterpret_cast<T*>(a.act);
    const int tiles = n / 8;
    const int items = nact * tiles;
    G.setup(dec_pick_w(items, d / S));
    for (int u = G.gid; u < items; u += G.ngroups) {
      const int e = L.active[u / tiles], j0 = (u % tiles) * 8;
      const int c = __builtin_amdgcn_readfirstlane(a.cnt[e]);
      const int32_t* lst = a.list + (int64_t)e * T_;
      const T* wrow = r16 < 8 ? Wg + ((int64_t)e * n + j0 + r16) * d : Wu + ((int64_t)e * n + j0 + r16 - 8) * d;
      const int groups = (c + 15) / 16;
      for (int g0 = 0; g0 < groups; g0 += DEC_NG) {
        const int ng = min(DEC_NG, groups - g0);
        const T* xr[DEC_NG];
#pragma unroll
        for (int g = 0; g < DEC_NG; ++g) xr[g] = X + (int64_t)(lst[min((g0 + g) * 16 + r16, c - 1)] / K) * d;
        dec_group_tile<T>(G, L, wrow, xr, ng, 0, d / S, [&](const f32x4* v) {
          for (int g = 0; g < ng; ++g) {
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = __shfl_xor(v[g][i], 32, 64);
            const int slot = (g0 + g) * 16 + r16;
            if (lane < 32 && slot < c) {  // lanes < 32: gate rows 4q + i, their up rows in lane + 32
              f32x4 h;
#pragma unroll
              for (int i = 0; i < 4; ++i) h[i] = v[g][i] * sigmoid_f32(v[g][i]) * o[i];
              dec_store4<T>(act + (int64_t)lst[slot] * n + j0 + 4 * q, h);
            }
          }
        });
      }
    }
  }
  if (!dec_grid_barrier(bar, a.spin_limit, L)) return;

  // ---- D: down tiles (16 output columns) -> y[pair] ----
  {
    const T* Wd = reinterpret_cast<const T*>(a.W_down);
    const T* act = reinterpret_cast<const T*>(a.act);
    const int tiles = d / 16;
    const int items = nact * tiles;
    G.setup(dec_pick_w(items, n / S));
    for (int u = G.gid; u < items; u += G.ngroups) {
      const int e = L.active[u / tiles], col0 = (u % tiles) * 16;
      const int c = __builtin_amdgcn_readfirstlane(a.cnt[e]);
      const int32_t* lst = a.list + (int64_t)e * T_;
      const T* wrow = Wd + ((int64_t)e * d + col0 + r16) * n;
      const int groups = (c + 15) / 16;
      for (int g0 = 0; g0 < groups; g0 += DEC_NG) {
        const int ng = min(DEC_NG, groups - g0);
        const T* xr[DEC_NG];
#pragma unroll
        for (int g = 0; g < DEC_NG; ++g) xr[g] = act + (int64_t)lst[min((g0 + g) * 16 + r16, c - 1)] * n;
        dec_group_tile<T>(G, L, wrow, xr, ng, 0, n / S, [&](const f32x4* v) {
          for (int g = 0; g < ng; ++g) {
            const int slot = (g0 + g) * 16 + r16;
            if (slot < c) *reinterpret_cast<f32x4*>(a.y + (int64_t)lst[slot] * d + col0 + 4 * q) = v[g];
          }
        });
      }
    }
  }
  if (!dec_grid_barrier(bar, a.spin_limit, L)) return;

  // ---- E: combine in ascending expert order, 4 columns per thread ----
  {
    const int chunks = (d + 4 * DEC_THREADS - 1) / (4 * DEC_THREADS);
    for (int u = blockIdx.x; u < T_ * chunks; u += gridDim.x) {
      const int t = u / chunks, c0 = (u % chunks) * 4 * DEC_THREADS + 4 * tid;
      // the token's experts (distinct, uniform over the workgroup) ranked by id: kb[r] is the k
      // of the r-th smallest
      int ids[16], kb[16];
#pragma unroll
      for (int k = 0; k < 16; ++k)
        ids[k] = k < K ? __builtin_amdgcn_readfirstlane(a.topk_idx[(int64_t)t * K + k]) : 0x7fffffff;
      int prev = -1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int best = 0x7fffffff, b = 0;
#pragma unroll
        for (int k = 0; k < 16; ++k)
          if (ids[k] > prev && ids[k] < best) {
            best = ids[k];
            b = k;
          }
        kb[r] = b;
        prev = best;
      }
      if (c0 < d) {
        f32x4 yv[16];
        float wv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (r < K) {
            const int64_t p = (int64_t)t * K + kb[r];
            wv[r] = a.topk_w[p];
            yv[r] = *reinterpret_cast<const f32x4*>(a.y + p * d + c0);
          }
        }
        f32x4 s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (r < K) s += wv[r] * yv[r];
        dec_store4<T>(reinterpret_cast<T*>(a.out) + (int64_t)t * d + c0, s);
      }
    }
  }
}

static size_t dec_align(size_t b) { return (b + 255) / 256 * 256; }

size_t decode_workspace_bytes(int64_t T, int64_t d, int64_t n, int E, int K) {
  return dec_align(8) + dec_align((size_t)E * 4) + dec_align((size_t)E * T * 4) +
         dec_align((size_t)T * K * n * 4) + dec_align((size_t)T * K * d * 4);
}

static long long g_dec_spin_limit = 1ll << 20;  // about a second of polling
// Grid size per device and dtype (0 until the first call on that device computes it).
constexpr int DEC_MAX_DEVICES = 64;
static std::atomic<int> g_dec_grid[DEC_MAX_DEVICES][2];

long long decode_set_spin_limit(long long limit) {
  const long long prev = g_dec_spin_limit;
  g_dec_spin_limit = limit;
  return prev;
}

hipError_t decode_read_status(hipStream_t st, int* failed) {
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return e;
  int v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_dec_status), sizeof v, 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  *failed = v;
  if (v) {
    const int zero = 0;
    e = hipMemcpyToSymbol(HIP_SYMBOL(g_dec_status), &zero, sizeof zero, 0, hipMemcpyHostToDevice);
  }
  return e;
}

hipError_t launch_decode(const Shape& s, const void* X, const void* W_r, const float* bias,
                         const void* W_gate, const void* W_up, const void* W_down, float* logits,
                         int32_t* topk_idx, float* topk_w, void* out, void* ws, hipStream_t st) {
  DecodeArgs a;
  a.X = X; a.W_r = W_r; a.bias = bias; a.W_gate = W_gate; a.W_up = W_up; a.W_down = W_down;
  a.logits = logits; a.topk_idx = topk_idx; a.topk_w = topk_w; a.out = out;
  char* w = static_cast<char*>(ws);
  a.bar = reinterpret_cast<unsigned long long*>(w);
  w += dec_align(8);
  a.cnt = reinterpret_cast<int32_t*>(w);
  w += dec_align((size_t)s.E * 4);
  a.list = reinterpret_cast<int32_t*>(w);
  w += dec_align((size_t)s.E * s.T * 4);
  a.act = w;  // element type; sized for fp32
  w += dec_align((size_t)s.T * s.K * s.n * 4);
  a.y = reinterpret_cast<float*>(w);
  a.T = (int)s.T; a.d = (int)s.d; a.n = (int)s.n; a.E = s.E; a.K = s.K;
  a.spin_limit = g_dec_spin_limit;
  const void* fn = s.bf16 ? reinterpret_cast<const void*>(&k_decode<bf16>)
                          : reinterpret_cast<const void*>(&k_decode<float>);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  // every workgroup must be resident at once for the grid barriers: the grid is the device's CU
  // count times the kernel's occupancy, queried once per device and dtype
  if (dev < 0 || dev >= DEC_MAX_DEVICES) return hipErrorInvalidDevice;
  std::atomic<int>& cached = g_dec_grid[dev][s.bf16 ? 1 : 0];
  int grid = cached.load(std::memory_order_relaxed);
  if (grid == 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, DEC_THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
    grid = cus * per_cu;
    cached.store(grid, std::memory_order_relaxed);
  }
  k_dec_clear<<<1, 256, 0, st>>>(a.bar, a.cnt, s.E);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // A plain launch: a grid of at most one full CU's worth of workgroups per CU is placed whole on
  // a device that runs nothing else, and the barriers' bounded wait turns the case where it
  // cannot be (other work holding CUs past the bound) into a reported failure.  The
  // cooperative launch gives the same guarantee up front but costs about 20 us more per call,
  // a third of a small decode step.
  void* params[] = {&a};
  return hipLaunchKernel(fn, dim3(grid), dim3(DEC_THREADS), params, 0u, st);
}

}  // namespace moe

// Routing kernels: top-K + softmax, per-expert membership bitmap and counts, token rounding,
// offsets and the (token, expert) -> row placement.
//
// Pages: cloud.baidu.com "工作原理" (gate network, top_k), apxml.com "自定义核与核融合" steps 1-2,
// SonicMoE page optimization 3 (token rounding), ThunderEP article section 2.2.2 (int32 row index
// lists).  Design for gfx950: selection by DPP reductions within a 16-lane row per token (E <= 256)
// or a whole wave per token (larger E), no LDS round trips; the membership of every
// (token, expert) pair lives in a bitmap bits[E][ceil(T/32)] built in LDS per block, so that
// per-expert counts, in-expert ranks (rows ordered by token id) and token rounding are popcounts
// and scans over 32-bit words; no atomics touch global memory and every result is deterministic.
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------------------------------------
// top-K: one wave per token, 16 waves per block of 64 tokens.  Lane i holds the order keys of
// logits e = i + 64 j.  Each of K rounds picks the largest key among the candidates still in
// play (a wave maximum through DPP row shifts and row broadcasts, no LDS traffic) and, among the
// candidates holding it, the lowest expert id (ballots scanned in ascending e) -- the order of
// logit descending, then expert id ascending.  The winners' logits are re-read for the softmax
// over the K of them, and the winners set their bit in the block's LDS bitmap (bitwise OR is
// order independent).
// ---------------------------------------------------------------------------------------------
constexpr int TOPK_TOKENS_PER_BLOCK = 64;  // two 32-bit bitmap words per expert per block
constexpr int TOPK_THREADS = 1024;

// Order-preserving integer key of an fp32 logit: a > b as floats <=> key(a) > key(b), -0.0 and
// +0.0 share a key, and NaN takes the smallest key (it ranks below every number).  Selecting on
// keys makes every comparison a total order, so all 64 lanes of a wave agree on each winner
// even for NaN inputs (float comparisons with NaN are not an order, and lanes could then pick
// the same expert twice).
__device__ __forceinline__ uint32_t order_key(float x) {
  if (x != x) return 0u;
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// The float an order key came from: exact for every number (-0.0 comes back as +0.0, which no
// difference or exponential below tells apart); key 0 comes back as a NaN.
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Logit e of token t: logits[t][e], plus, after a split router GEMM, its SK - 1 partial products
// in slice order; the sum is written back so that the logits output holds the final values.
__device__ __forceinline__ float token_logit(float* __restrict__ logits, const float* __restrict__ part, int SK,
                                            int T, int E, int t, int e) {
  const int64_t i = (int64_t)t * E + e;
  float v = logits[i];
  if (SK > 1) {
    for (int q = 0; q < SK - 1; ++q) v += part[(int64_t)q * T * E + i];
    logits[i] = v;
  }
  return v;
}

// keysT (token rounding only, else null): the order keys transposed, keysT[e][t], for the rounding
// kernel's per-expert scans.  With E <= TOPK_STAGE_E the block's keys are staged in LDS
// ([e][65], conflict-free) and written out as 64-token rows; otherwise each lane stores its own.
constexpr int TOPK_STAGE_E = 192;  // E * (2 + 65) words stay within the default 64 KiB of dynamic LDS
template <int EPL>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk(float* __restrict__ logits, const float* __restrict__ part,
                                                       int SK, int T, int E,
                                                       int K, int W, int32_t* __restrict__ topk_idx,
                                                       float* __restrict__ topk_w,
                                                       uint32_t* __restrict__ bits,
                                                       uint32_t* __restrict__ keysT) {
  extern __shared__ uint32_t sbits[];  // [E][2], then (keysT staged) [E][65] keys
  uint32_t* skeys = sbits + 2 * E;
  const bool stage = keysT && E <= TOPK_STAGE_E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TOPK_TOKENS_PER_BLOCK;
  for (int i = threadIdx.x; i < 2 * E; i += blockDim.x) sbits[i] = 0u;
  __syncthreads();
  for (int tt = wave; tt < TOPK_TOKENS_PER_BLOCK; tt += TOPK_THREADS / 64) {
    const int t = t0 + tt;
    if (t >= T) break;
    uint32_t key[EPL];
    uint32_t alive = 0;  // bit j: candidate e = lane + 64 j still in play
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      key[j] = e < E ? order_key(token_logit(logits, part, SK, T, E, t, e)) : 0u;
      alive |= e < E ? (1u << j) : 0u;
      if (keysT && e < E) {
        if (stage) skeys[e * 65 + tt] = key[j];
        else keysT[(int64_t)e * T + t] = key[j];
      }
    }
    int my_e = 0;
    uint32_t my_key = 0;
    for (int k = 0; k < K; ++k) {
      uint32_t lm = 0;  // NaN keys are 0 too; ties at 0 are settled below among live candidates
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if ((alive >> j) & 1u) lm = key[j] > lm ? key[j] : lm;
      const uint32_t kmax = wave_max_u32(lm);
      if (lane == k) my_key = kmax;
      int win = -1;  // lowest expert id holding kmax (uniform)
#pragma unroll
      for (int j = 0; j < EPL; ++j) {
        const uint64_t m = __builtin_amdgcn_ballot_w64(((alive >> j) & 1u) && key[j] == kmax);
        if (win < 0 && m != 0ull) win = 64 * j + (int)__builtin_ctzll(m);
      }
      win = __builtin_amdgcn_readfirstlane(win);
      if (lane == (win & 63)) alive &= ~(1u << (win >> 6));
      if (lane == k) my_e = win;
    }
    const float my_v = lane < K ? key_value(my_key) : 0.0f;  // the winner's logit, from its key
    const float vmax = __shfl(my_v, 0, 64);
    const float ex = lane < K ? __expf(my_v - vmax) : 0.0f;
    const float s = wave_sum(ex);
    if (lane < K) {
      topk_idx[(int64_t)t * K + lane] = my_e;
      topk_w[(int64_t)t * K + lane] = ex / s;
      atomicOr(&sbits[my_e * 2 + (tt >> 5)], 1u << (tt & 31));
    }
  }
  __syncthreads();
  const int w0 = blockIdx.x * 2;
  for (int i = threadIdx.x; i < 2 * E; i += blockDim.x) {
    const int e = i >> 1, w = w0 + (i & 1);
    if (w < W) bits[(int64_t)e * W + w] = sbits[i];
  }
  if (stage)
    for (int i = threadIdx.x; i < E * 64; i += blockDim.x) {
      const int e = i >> 6, c = i & 63;
      if (t0 + c < T) keysT[(int64_t)e * T + t0 + c] = skeys[e * 65 + c];
    }
}

// ---------------------------------------------------------------------------------------------
// top-K for E <= 256: four tokens per wave, one 16-lane row of the wave per token (the same 64
// tokens and 16 waves per block).  Lane i of a row holds the order keys of experts e = i + 16 j,
// j < EPG.  A round takes the row's largest live key (rotations by 1, 2, 4 and 8 lanes within the
// row leave the maximum in every lane, one v_max_u32 with a DPP operand each), then the lowest
// expert id holding it (the same with minima over each lane's lowest candidate) -- the same
// order as the wave-per-token kernel, with a quarter of its instructions per token.
// ---------------------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t row_ror_max(uint32_t v) {
  const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
  return v > x ? v : x;
}
template <int CTRL>
__device__ __forceinline__ uint32_t row_ror_min(uint32_t v) {
  const uint32_t x = (uint32_t)__builtin_amdgcn_update_dpp(-1, (int)v, CTRL, 0xf, 0xf, true);
  return v < x ? v : x;
}
__device__ __forceinline__ uint32_t row16_max(uint32_t v) {
  v = row_ror_max<0x121>(v);  // row_ror:1
  v = row_ror_max<0x122>(v);  // row_ror:2
  v = row_ror_max<0x124>(v);  // row_ror:4
  return row_ror_max<0x128>(v);  // row_ror:8
}
__device__ __forceinline__ uint32_t row16_min(uint32_t v) {
  v = row_ror_min<0x121>(v);
  v = row_ror_min<0x122>(v);
  v = row_ror_min<0x124>(v);
  return row_ror_min<0x128>(v);
}

template <int EPG>
__global__ __launch_bounds__(TOPK_THREADS) void k_topk_g(float* __restrict__ logits, const float* __restrict__ part,
                                                         int SK, int T, int E,
                                                         int K, int W, int32_t* __restrict__ topk_idx,
                                                         float* __restrict__ topk_w,
                                                         uint32_t* __restrict__ bits,
                                                         uint32_t* __restrict__ keysT) {
  extern __shared__ uint32_t sbits[];  // [E][2], then (keysT staged) [E][65] keys
  uint32_t* skeys = sbits + 2 * E;
  const bool stage = keysT && E <= TOPK_STAGE_E;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int i = lane & 15;
  const int tt = wave * 4 + (lane >> 4);  // the row's token within the block
  const int t0 = blockIdx.x * TOPK_TOKENS_PER_BLOCK;
  const int t = t0 + tt;
  for (int x = threadIdx.x; x < 2 * E; x += blockDim.x) sbits[x] = 0u;
  __syncthreads();
  if (t < T) {  // uniform over the row, so every DPP source lane is active
    uint32_t key[EPG];
    uint32_t alive = 0;  // bit j: candidate e = i + 16 j still in play
#pragma unroll
    for (int j = 0; j < EPG; ++j) {
      const int e = i + 16 * j;
      key[j] = e < E ? order_key(token_logit(logits, part, SK, T, E, t, e)) : 0u;
      alive |= e < E ? (1u << j) : 0u;
      if (keysT && e < E) {
        if (stage) skeys[e * 65 + tt] = key[j];
        else keysT[(int64_t)e * T + t] = key[j];
      }
    }
    int my_e = 0;
    uint32_t my_key = 0;
    for (int k = 0; k < K; ++k) {
      uint32_t lm = 0;  // NaN keys are 0 too; ties at 0 are settled below among live candidates
#pragma unroll
      for (int j = 0; j < EPG; ++j)
        if ((alive >> j) & 1u) lm = key[j] > lm ? key[j] : lm;
      const uint32_t kmax = row16_max(lm);
      if (i == k) my_key = kmax;
      uint32_t cand = 0xffffffffu;  // this lane's lowest expert id holding kmax
#pragma unroll
      for (int j = EPG - 1; j >= 0; --j)
        if (((alive >> j) & 1u) && key[j] == kmax) cand = (uint32_t)(i + 16 * j);
      const int win = (int)row16_min(cand);
      if (i == (win & 15)) alive &= ~(1u << (win >> 4));
      if (i == k) my_e = win;
    }
    const float my_v = i < K ? key_value(my_key) : 0.0f;  // the winner's logit, from its key
    const float vmax = __shfl(my_v, lane & ~15, 64);
    const float ex = i < K ? __expf(my_v - vmax) : 0.0f;
    float s = ex;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);  // the same sum in every lane of the row
    if (i < K) {
      topk_idx[(int64_t)t * K + i] = my_e;
      topk_w[(int64_t)t * K + i] = ex / s;
      atomicOr(&sbits[my_e * 2 + (tt >> 5)], 1u << (tt & 31));
    }
  }
  __syncthreads();
  const int w0 = blockIdx.x * 2;
  for (int x = threadIdx.x; x < 2 * E; x += blockDim.x) {
    const int e = x >> 1, w = w0 + (x & 1);
    if (w < W) bits[(int64_t)e * W + w] = sbits[x];
  }
  if (stage)
    for (int x = threadIdx.x; x < E * 64; x += blockDim.x) {
      const int e = x >> 6, c = x & 63;
      if (t0 + c < T) keysT[(int64_t)e * T + t0 + c] = skeys[e * 65 + c];
    }
}

// ---------------------------------------------------------------------------------------------
// Block-wide exclusive scan helper (256 threads).  Returns the exclusive prefix of `x` and the
// block total.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ int block_exscan_256(int x, int* total, int* sh /*[4]*/) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    base += (w < wave) ? sh[w] : 0;
    tot += sh[w];
  }
  __syncthreads();
  *total = tot;
  return base + inc - x;
}

// Per expert (one block each): counts[e] = popcount of its bitmap row, and the exclusive prefix
// of popcounts per word, which is the rank of a member token among the expert's earlier tokens.
__global__ __launch_bounds__(256) void k_count(const uint32_t* __restrict__ bits, int W,
                                               int32_t* __restrict__ wprefix,
                                               int32_t* __restrict__ counts) {
  __shared__ int sh[4];
  const int e = blockIdx.x;
  const uint32_t* b = bits + (int64_t)e * W;
  int32_t* p = wprefix + (int64_t)e * W;
  int carry = 0;
  for (int w0 = 0; w0 < W; w0 += 256) {
    const int w = w0 + threadIdx.x;
    const int c = w < W ? __popc(b[w]) : 0;
    int tot;
    const int ex = block_exscan_256(c, &tot, sh);
    if (w < W) p[w] = carry + ex;
    carry += tot;
  }
  if (threadIdx.x == 0) counts[e] = carry;
}

// ---------------------------------------------------------------------------------------------
// Token rounding, one 1024-thread block per expert.  Direction: NEAREST adds when 2r >= M, UP
// always, DOWN never, STOCHASTIC when the expert's caller-drawn word w satisfies w M < r 2^32
// (probability r / M: the expected count stays c); an addition past T tokens drops instead.
// Key of token t for expert e, larger = chosen first:
//   adding  (best non-members): (ord(L[t,e]) << 32) | ~t      -> larger logit, then lower t
//   dropping (worst members):   (~ord(L[t,e]) << 32) | t      -> smaller logit, then higher t
// ord() is order_key (-0.0 folded onto +0.0, NaN lowest).  Keys are unique (t is), so the set of
// the `amount` largest keys is unique; it is found by an 8-pass radix select over 8-bit digits
// and the bitmap row is rewritten.  Most candidates share their top digits (those of the logit's
// sign and exponent), so the lanes of a wave that hit its first participant's bin add their
// count with one LDS atomic; one wave then locates the digit with a suffix scan.  Once every
// candidate left under the chosen prefix is taken, the threshold is their minimum and the
// remaining passes are skipped.
// When T <= TR_LDS_TOKENS the expert's logit keys and bitmap row are cached in LDS.
// ---------------------------------------------------------------------------------------------
constexpr int TR_THREADS = 1024;
constexpr int TR_LDS_TOKENS = 32768;

__host__ __device__ __forceinline__ size_t tr_lds_bytes(int64_t T, int W) {
  return T <= TR_LDS_TOKENS ? (size_t)(T + W) * 4 : 0;
}

__global__ __launch_bounds__(TR_THREADS) void k_token_round(const float* __restrict__ logits, int T,
                                                           int E, int W, int M, int mode,
                                                           const uint32_t* __restrict__ round_rand,
                                                           uint32_t* __restrict__ bits,
                                                           const int32_t* __restrict__ counts,
                                                           const uint32_t* __restrict__ keysT) {
  extern __shared__ uint32_t s_dyn[];  // cached: [T] logit keys, then [W] bitmap words
  __shared__ int hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ unsigned long long s_min;
  __shared__ int s_need;
  __shared__ bool s_all;
  const int e = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int c = counts[e];
  const int r = c % M;
  if (r == 0) return;
  bool add;
  if (mode == 1) add = 2 * r >= M;
  else if (mode == 2) add = true;
  else if (mode == 4) add = (uint64_t)round_rand[e] * (uint64_t)M < ((uint64_t)r << 32);  // P = r / M
  else add = false;
  if (add && (int64_t)c + (M - r) > T) add = false;
  const int amount = add ? (M - r) : r;
  const bool cached = T <= TR_LDS_TOKENS;
  uint32_t* brow = bits + (int64_t)e * W;
  uint32_t* s_ord = s_dyn;
  uint32_t* s_bits = s_dyn + T;
  if (cached) {
#pragma unroll 8
    for (int t = threadIdx.x; t < T; t += TR_THREADS)
      s_ord[t] = keysT ? keysT[(int64_t)e * T + t] : order_key(logits[(int64_t)t * E + e]);
    for (int w = threadIdx.x; w < W; w += TR_THREADS) s_bits[w] = brow[w];
    __syncthreads();
  }
  auto key_of = [&](int t, bool& cand) -> uint64_t {
    const uint32_t word = cached ? s_bits[t >> 5] : brow[t >> 5];
    const bool mem = (word >> (t & 31)) & 1u;
    cand = add ? !mem : mem;
    const uint32_t o = cached ? s_ord[t] : keysT ? keysT[(int64_t)e * T + t] : order_key(logits[(int64_t)t * E + e]);
    return add ? (((uint64_t)o << 32) | (uint32_t)(~(uint32_t)t))
               : (((uint64_t)(~o) << 32) | (uint32_t)t);
  };
  const int iters = (T + TR_THREADS - 1) / TR_THREADS;  // uniform trip count: ballots see every lane
  uint64_t prefix = 0;  // digits fixed so far (high bits)
  int need = amount;    // how many keys >= threshold still to take within the current prefix
  for (int pass = 0; pass < 8; ++pass) {
    const int shift = 56 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += TR_THREADS) hist[i] = 0;
    __syncthreads();
    const uint64_t hi_mask = pass == 0 ? 0ull : (~0ull << (shift + 8));
    for (int it = 0; it < iters; ++it) {
      const int t = it * TR_THREADS + threadIdx.x;
      bool part = false;
      int dig = 0;
      if (t < T) {
        bool cand;
        const uint64_t k = key_of(t, cand);
        part = cand && (k & hi_mask) == prefix;
        dig = (int)((k >> shift) & 255);
      }
      const uint64_t act = __builtin_amdgcn_ballot_w64(part);
      if (act) {  // uniform: the first participant's bin takes one merged atomic
        const int leader = (int)__builtin_ctzll(act);
        const int ld = __shfl(dig, leader, 64);
        const uint64_t same = __builtin_amdgcn_ballot_w64(part && dig == ld);
        if (lane == leader) atomicAdd(&hist[ld], (int)__builtin_popcountll(same));
        else if (part && dig != ld) atomicAdd(&hist[dig], 1);
      }
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      // lane l holds bins 4l .. 4l+3; suffix sums over lanes find the digit where the running
      // count (from the top bin down) first reaches `need`.
      int h[4], s4 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = hist[4 * lane + j];
        s4 += h[j];
      }
      int suf = s4;  // sum of s4 over lanes lane .. 63
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_down(suf, o, 64);
        if (lane + o < 64) suf += v;
      }
      const int above = suf - s4;  // candidates in bins above 4 lane + 3
      if (above < need && need <= suf) {
        int acc = above, dsel = 4 * lane;
        for (int j = 3; j >= 0; --j) {
          if (acc + h[j] >= need) {
            dsel = 4 * lane + j;
            break;
          }
          acc += h[j];
        }
        s_prefix = prefix | ((uint64_t)dsel << shift);
        s_need = need - acc;
        s_all = (need - acc) == h[dsel - 4 * lane];
      }
    }
    __syncthreads();
    prefix = s_prefix;
    need = s_need;
    const bool all = s_all;
    __syncthreads();
    if (all && pass < 7) {
      // every candidate under the new prefix is taken: the threshold is the smallest of them
      const uint64_t pmask = ~0ull << shift;
      if (threadIdx.x == 0) s_min = ~0ull;
      __syncthreads();
      for (int t = threadIdx.x; t < T; t += TR_THREADS) {
        bool cand;
        const uint64_t k = key_of(t, cand);
        if (cand && (k & pmask) == prefix) atomicMin(&s_min, k);
      }
      __syncthreads();
      prefix = s_min;
      break;
    }
  }
  // prefix is now the smallest chosen key: every candidate with key >= prefix flips membership.
  // Each word is owned by one thread, which reads only its own word's bits.
  const uint64_t thr = prefix;
  for (int w = threadIdx.x; w < W; w += TR_THREADS) {
    uint32_t word = cached ? s_bits[w] : brow[w];
    const uint32_t orig = word;
    for (int b = 0; b < 32; ++b) {
      const int t = w * 32 + b;
      if (t >= T) break;
      const bool mem = (orig >> b) & 1u;
      const bool cand = add ? !mem : mem;
      const uint32_t o = cached ? s_ord[t] : keysT ? keysT[(int64_t)e * T + t] : order_key(logits[(int64_t)t * E + e]);
      const uint64_t k = add ? (((uint64_t)o << 32) | (uint32_t)(~(uint32_t)t))
                             : (((uint64_t)(~o) << 32) | (uint32_t)t);
      if (cand && k >= thr) word ^= (1u << b);
    }
    brow[w] = word;
  }
}

// expert_off = exclusive scan of counts (E <= 1024, one block of 1024 threads); meta[0] = R.
__global__ __launch_bounds__(1024) void k_offsets(const int32_t* __restrict__ counts, int E,
                                                  int32_t* __restrict__ expert_off,
                                                  int32_t* __restrict__ meta) {
  __shared__ int sh[16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = threadIdx.x < E ? counts[threadIdx.x] : 0;
  int inc = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(inc, o, 64);
    if (lane >= o) inc += y;
  }
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    base += (w < wave) ? sh[w] : 0;
    tot += sh[w];
  }
  if (threadIdx.x < E) expert_off[threadIdx.x] = base + inc - x;
  if (threadIdx.x == 0) {
    expert_off[E] = tot;
    meta[0] = tot;
  }
}

// Stage the bitmap words of a 256-token block (8 words per expert) in LDS: sb[e * 8 + j] is word
// blockIdx.x * 8 + j of expert e (0 past the end).  Coalesced 32-byte pieces replace E strided
// loads per token.
__device__ __forceinline__ void stage_block_bits(const uint32_t* __restrict__ bits, int E, int W,
                                                 uint32_t* sb) {
  const int w0 = blockIdx.x * 8;
  for (int i = threadIdx.x; i < E * 8; i += blockDim.x) {
    const int e = i >> 3, w = w0 + (i & 7);
    sb[i] = w < W ? bits[(int64_t)e * W + w] : 0u;
  }
  __syncthreads();
}

// Token rounding: the number of final rows of each group of 32 tokens (one bitmap word) ->
// grp[g + 1], scanned afterwards by k_tok_scan over the groups.  256 threads per block, one token
// each; dynamic LDS E * 8 words.
__global__ __launch_bounds__(256) void k_tok_count(const uint32_t* __restrict__ bits, int T, int E,
                                                   int W, int32_t* __restrict__ grp) {
  extern __shared__ uint32_t sb[];
  stage_block_bits(bits, E, W, sb);
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int wl = threadIdx.x >> 5;
  int c = 0;
  if (t < T)
    for (int e = 0; e < E; ++e) c += (sb[e * 8 + wl] >> (t & 31)) & 1u;
#pragma unroll
  for (int o = 1; o < 32; o <<= 1) c += __shfl_xor(c, o, 32);
  if ((threadIdx.x & 31) == 0 && t < T) grp[(t >> 5) + 1] = c;
}

// In-place scan: tok_off[1..T] holds counts; afterwards tok_off[t] = sum of counts before t.
// One block of 1024 threads, sequential over chunks of 1024 * 8 tokens.
__global__ __launch_bounds__(1024) void k_tok_scan(int T, int32_t* __restrict__ tok_off) {
  __shared__ int sh[16];
  __shared__ int s_carry;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) s_carry = 0;
  __syncthreads();
  constexpr int PER = 8;
  for (int base0 = 0; base0 < T; base0 += 1024 * PER) {
    int v[PER];
    int loc = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = base0 + threadIdx.x * PER + i;
      v[i] = t < T ? tok_off[t + 1] : 0;
      loc += v[i];
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(inc, o, 64);
      if (lane >= o) inc += y;
    }
    if (lane == 63) sh[wave] = inc;
    __syncthreads();
    int wb = 0, tot = 0;
    for (int w = 0; w < 16; ++w) {
      wb += (w < wave) ? sh[w] : 0;
      tot += sh[w];
    }
    int run = s_carry + wb + inc - loc;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = base0 + threadIdx.x * PER + i;
      run += v[i];
      if (t < T) tok_off[t + 1] = run;
    }
    __syncthreads();
    if (threadIdx.x == 0) s_carry += tot;
    __syncthreads();
  }
  if (threadIdx.x == 0) tok_off[0] = 0;
}

// ---------------------------------------------------------------------------------------------
// Placement of plain top-K: one thread per token.  The token's K ids in ascending order (a bitonic
// network over KM >= K registers, padded with INT_MAX, every index fixed at compile time so that
// nothing goes to scratch memory); gate weights = softmax of its K logits; row of (t, e) =
// expert_off[e] + (members of e before t), a popcount.
// ---------------------------------------------------------------------------------------------
template <int N>
__device__ __forceinline__ void bitonic_sort_i32(int (&a)[N]) {
#pragma unroll
  for (int k = 2; k <= N; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int l = i ^ j;
        if (l > i) {
          const int x = a[i], y = a[l];
          const bool sw = ((i & k) == 0) ? (x > y) : (x < y);
          a[i] = sw ? y : x;
          a[l] = sw ? x : y;
        }
      }
}

template <int KM>
__global__ __launch_bounds__(256) void k_place(const float* __restrict__ logits, int T, int E,
                                               int K, int W, const int32_t* __restrict__ topk_idx,
                                               const uint32_t* __restrict__ bits,
                                               const int32_t* __restrict__ wprefix,
                                               const int32_t* __restrict__ expert_off,
                                               int32_t* __restrict__ tok_off,
                                               int32_t* __restrict__ row_token,
                                               float* __restrict__ row_w,
                                               int32_t* __restrict__ tok_row) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const int base = t * K;  // plain top-K: every token has K rows
  tok_off[t] = base;
  if (t == T - 1) tok_off[T] = T * K;
  const float* L = logits + (int64_t)t * E;
  const int w = t >> 5;
  const uint32_t below = (1u << (t & 31)) - 1u;
  int ids[KM];
  float lv[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) ids[k] = k < K ? topk_idx[(int64_t)t * K + k] : INT_MAX;
  bitonic_sort_i32(ids);
  // every load below is issued for all KM slots (slots k >= K read expert 0 and are ignored), so
  // that they go out together instead of one dependent round trip per slot
  int rows[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    const int e = k < K ? ids[k] : 0;
    lv[k] = L[e];
    rows[k] = expert_off[e] + wprefix[(int64_t)e * W + w] + __popc(bits[(int64_t)e * W + w] & below);
  }
  // (an empty asm that takes the rows and logits keeps the compiler from sinking their loads
  // towards their conditional uses below, one round trip each)
  if constexpr (KM <= 8) {  // (at 16 slots the pinned values crowd the registers)
#pragma unroll
    for (int k = 0; k < KM; ++k) asm volatile("" : "+v"(rows[k]), "+v"(lv[k]));
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) lv[k] = k < K ? lv[k] : -INFINITY;
  float m = lv[0];
#pragma unroll
  for (int k = 1; k < KM; ++k)
    if (k < K) m = fmaxf(m, lv[k]);
  float s = 0.0f;
#pragma unroll
  for (int k = 0; k < KM; ++k)
    if (k < K) s += __expf(lv[k] - m);
  const float inv = 1.0f / s;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= K) break;
    const int row = rows[k];
    row_token[row] = t;
    row_w[row] = __expf(lv[k] - m) * inv;
    tok_row[base + k] = row;
  }
}

// Placement after token rounding: a token's final experts are the set bits of its bitmap column
// (any number of them).  Eight lanes per token, 32 tokens (one bitmap word per expert) per block of
// 256 threads: lane j of a token takes experts j * EP .. j * EP + EP - 1 (EP = ceil(E / 8)), so the
// lanes' member lists, concatenated in lane order, are in ascending expert id.  The token's
// logit maximum and softmax sum are combined over its eight lanes; each member's place among the
// token's rows is the lane's exclusive prefix of member counts plus its rank in the lane.  The
// token's first row is the group prefix (grp, scanned over groups of 32 tokens) plus the
// exclusive scan of the counts of the group's earlier tokens.
constexpr int PR_CHUNK = 16;  // experts per unrolled chunk of a lane's range
__global__ __launch_bounds__(256) void k_place_rounded(const float* __restrict__ logits, int T, int E, int W,
                                                       const uint32_t* __restrict__ bits,
                                                       const int32_t* __restrict__ wprefix,
                                                       const int32_t* __restrict__ expert_off,
                                                       const int32_t* __restrict__ grp,
                                                       int32_t* __restrict__ tok_off,
                                                       int32_t* __restrict__ row_token,
                                                       float* __restrict__ row_w,
                                                       int32_t* __restrict__ tok_row) {
  extern __shared__ uint32_t sw[];  // [E]: this group's bitmap word of each expert
  __shared__ int scnt[32];
  const int g = blockIdx.x;          // group of 32 tokens = bitmap word g
  for (int e = threadIdx.x; e < E; e += 256) sw[e] = bits[(int64_t)e * W + g];
  __syncthreads();
  const int tt = threadIdx.x >> 3, sub = threadIdx.x & 7;
  const int t = g * 32 + tt;
  const bool live = t < T;
  const int EP = (E + 7) / 8;
  const int e_lo = sub * EP, e_hi = min(E, e_lo + EP);
  const uint32_t below = (1u << tt) - 1u;
  const float* L = logits + (int64_t)(live ? t : 0) * E;
  // members of this lane and the lane's logit maximum
  int c = 0;
  float m = -INFINITY;
  for (int e0 = e_lo; e0 < e_hi; e0 += PR_CHUNK) {
    uint32_t mw = 0;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b)
      if (live && e0 + b < e_hi) mw |= ((sw[e0 + b] >> tt) & 1u) << b;
    c += __popc(mw);
    float v[PR_CHUNK];
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b) v[b] = ((mw >> b) & 1u) ? L[e0 + b] : -INFINITY;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b)
      if ((mw >> b) & 1u) m = fmaxf(m, v[b]);
  }
  // combine over the token's eight lanes (xor partners stay inside the aligned group of 8)
  int cnt = c, pre = c;
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) {
    m = fmaxf(m, __shfl_xor(m, o, 64));
    cnt += __shfl_xor(cnt, o, 64);
    const int up = __shfl_up(pre, o, 8);
    if (sub >= o) pre += up;
  }
  pre -= c;  // exclusive prefix of member counts over the token's lanes
  // token offsets: group prefix + exclusive scan over the group's tokens
  if (sub == 0) scnt[tt] = live ? cnt : 0;
  __syncthreads();
  int before = 0;
  for (int j = 0; j < tt; ++j) before += scnt[j];
  const int base = grp[g] + before;
  if (live && sub == 0) {
    tok_off[t] = base;
    if (t == T - 1) tok_off[T] = base + cnt;
  }
  if (!live || cnt == 0) return;
  float s = 0.0f;
  for (int e0 = e_lo; e0 < e_hi; e0 += PR_CHUNK) {
    uint32_t mw = 0;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b)
      if (e0 + b < e_hi) mw |= ((sw[e0 + b] >> tt) & 1u) << b;
    float v[PR_CHUNK];
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b) v[b] = ((mw >> b) & 1u) ? L[e0 + b] : 0.0f;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b)
      if ((mw >> b) & 1u) s += __expf(v[b] - m);
  }
#pragma unroll
  for (int o = 1; o < 8; o <<= 1) s += __shfl_xor(s, o, 64);
  const float inv = 1.0f / s;
  int i = base + pre;
  for (int e0 = e_lo; e0 < e_hi; e0 += PR_CHUNK) {
    uint32_t mw = 0;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b)
      if (e0 + b < e_hi) mw |= ((sw[e0 + b] >> tt) & 1u) << b;
    float v[PR_CHUNK];
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b) v[b] = ((mw >> b) & 1u) ? L[e0 + b] : 0.0f;
#pragma unroll
    for (int b = 0; b < PR_CHUNK; ++b) {
      if (!((mw >> b) & 1u)) continue;
      const int e = e0 + b;
      const int row = expert_off[e] + wprefix[(int64_t)e * W + g] + __popc(sw[e] & below);
      row_token[row] = t;
      row_w[row] = __expf(v[b] - m) * inv;
      tok_row[i++] = row;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Host launcher for the whole routing plan from fp32 logits.
// ---------------------------------------------------------------------------------------------
// bits [E][W] | wprefix [E][W] | grp [W + 1] | (token rounding) keysT [E][T]
size_t route_workspace_bytes(int64_t T, int E, bool rounded) {
  const int64_t W = cdiv(T, 32);
  return align_up((size_t)E * W * 4, 256) * 2 + align_up((size_t)(W + 1) * 4, 256) +
         (rounded ? align_up((size_t)E * T * 4, 256) : 0);
}

hipError_t launch_route(float* logits, const float* part, int SK, int64_t T, int E, int K, int round_mode,
                        int tile_m, const uint32_t* round_rand, const PlanPtrs& p, void* ws, hipStream_t st) {
  const int W = (int)cdiv(T, 32);
  uint32_t* bits = static_cast<uint32_t*>(ws);
  int32_t* wprefix = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + align_up((size_t)E * W * 4, 256));
  int32_t* grp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + 2 * align_up((size_t)E * W * 4, 256));
  const bool rounded = round_mode != 0;
  uint32_t* keysT = rounded ? reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(grp) + align_up((size_t)(W + 1) * 4, 256))
                            : nullptr;
  const int nblk = (int)cdiv(T, TOPK_TOKENS_PER_BLOCK);
  const size_t lds = (size_t)E * 2 * sizeof(uint32_t) + (rounded && E <= TOPK_STAGE_E ? (size_t)E * 65 * 4 : 0);
#define MOE_TOPK(EPL) k_topk<EPL><<<nblk, TOPK_THREADS, lds, st>>>(logits, part, SK, (int)T, E, K, W, p.topk_idx, p.topk_w, bits, keysT)
#define MOE_TOPK_G(EPG) k_topk_g<EPG><<<nblk, TOPK_THREADS, lds, st>>>(logits, part, SK, (int)T, E, K, W, p.topk_idx, p.topk_w, bits, keysT)
  if (E <= 16) MOE_TOPK_G(1);
  else if (E <= 32) MOE_TOPK_G(2);
  else if (E <= 64) MOE_TOPK_G(4);
  else if (E <= 128) MOE_TOPK_G(8);
  else if (E <= 256) MOE_TOPK_G(16);
  else if (E <= 512) MOE_TOPK(8);
  else MOE_TOPK(16);
#undef MOE_TOPK_G
#undef MOE_TOPK
  k_count<<<E, 256, 0, st>>>(bits, W, wprefix, p.counts);
  if (rounded) {
    const size_t tr_lds = tr_lds_bytes(T, W);
    // dynamic LDS above 64 KiB must be opted into (per device; a cheap host call)
    const hipError_t ae = hipFuncSetAttribute(reinterpret_cast<const void*>(k_token_round),
                                              hipFuncAttributeMaxDynamicSharedMemorySize,
                                              (int)tr_lds_bytes(TR_LDS_TOKENS, TR_LDS_TOKENS / 32));
    if (ae != hipSuccess) return ae;
    k_token_round<<<E, TR_THREADS, tr_lds, st>>>(logits, (int)T, E, W, tile_m, round_mode, round_rand, bits,
                                                 p.counts, keysT);
    k_count<<<E, 256, 0, st>>>(bits, W, wprefix, p.counts);
  }
  k_offsets<<<1, 1024, 0, st>>>(p.counts, E, p.expert_off, p.meta);
  if (rounded) {
    k_tok_count<<<(int)cdiv(T, 256), 256, (size_t)E * 32, st>>>(bits, (int)T, E, W, grp);
    k_tok_scan<<<1, 1024, 0, st>>>(W, grp);
    k_place_rounded<<<W, 256, (size_t)E * 4, st>>>(logits, (int)T, E, W, bits, wprefix, p.expert_off, grp,
                                                   p.tok_off, p.row_token, p.row_w, p.tok_row);
  } else {
#define MOE_PLACE(KM) k_place<KM><<<(int)cdiv(T, 256), 256, 0, st>>>(logits, (int)T, E, K, W, p.topk_idx, bits, \
      wprefix, p.expert_off, p.tok_off, p.row_token, p.row_w, p.tok_row)
    if (K <= 2) MOE_PLACE(2);
    else if (K <= 4) MOE_PLACE(4);
    else if (K <= 8) MOE_PLACE(8);
    else MOE_PLACE(16);
#undef MOE_PLACE
  }
  return hipGetLastError();
}

}  // namespace moe

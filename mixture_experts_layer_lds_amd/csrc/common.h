// Shared device/host definitions of the gfx950 MoE kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// silu(g) = g * sigmoid(g); sigmoid via the hardware exp2 and the hardware reciprocal
// (v_rcp_f32, about 1 ulp: the correctly rounded quotient costs a ten-instruction sequence per
// element, which dominated the SwiGLU epilogues).  For g -> -inf, exp(-g) -> inf and the
// reciprocal goes to 0, which is the limit.
__device__ __forceinline__ float sigmoid_f32(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// Wave-wide reductions (64 lanes) through cross-lane shuffles.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
// Maximum of v over the 64 lanes, returned in every lane.  Within each row of 16 lanes, row
// shifts by 1, 2, 3, 4 (lanes 4-15) and 8 (lanes 8-15) leave the row's maximum in its lane 15;
// row broadcasts of lane 15 (into rows 1 and 3) and of lane 31 (into rows 2 and 3) then leave the
// wave's maximum in lane 63.  Lanes whose DPP source is off the row or masked read 0, the
// identity of an unsigned maximum, which lets the compiler fold each move into the maximum
// (one v_max_u32 with a DPP operand per step).
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v, uint32_t x) { return v > x ? v : x; }
template <int CTRL, int ROWS, int BANKS>
__device__ __forceinline__ uint32_t dpp_src(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, BANKS, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step(v, dpp_src<0x111, 0xf, 0xf>(v));  // row_shr:1
  v = dpp_max_step(v, dpp_src<0x112, 0xf, 0xf>(v));  // row_shr:2
  v = dpp_max_step(v, dpp_src<0x113, 0xf, 0xf>(v));  // row_shr:3
  v = dpp_max_step(v, dpp_src<0x114, 0xf, 0xe>(v));  // row_shr:4, lanes 4-15 of each row
  v = dpp_max_step(v, dpp_src<0x118, 0xf, 0xc>(v));  // row_shr:8, lanes 8-15 of each row
  v = dpp_max_step(v, dpp_src<0x142, 0xa, 0xf>(v));  // row_bcast:15 into rows 1 and 3
  v = dpp_max_step(v, dpp_src<0x143, 0xc, 0xf>(v));  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// 16-byte global load/store helpers (the pointer must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
// Streaming (non-temporal) variants for data read or written exactly once.
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// Elements of type T in one 16-byte chunk.
template <typename T> struct Vec { static constexpr int N = 16 / sizeof(T); };

// Unpack / pack a 16-byte chunk to/from fp32.
template <typename T> __device__ __forceinline__ void unpack16(u32x4 v, float* f);
template <> __device__ __forceinline__ void unpack16<float>(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
}
template <> __device__ __forceinline__ void unpack16<bf16>(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
template <typename T> __device__ __forceinline__ u32x4 pack16(const float* f);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
  return v;
}
// Two floats to two bf16 (round to nearest even) in one 32-bit word, lo in the low half: a
// two-element vector conversion, which gfx950 does in one instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float* f) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
  return v;
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Clamp a gathered index into [0, n): routing indices are always in range when they come from
// moe_route; the clamp keeps every gathered read in bounds even for a corrupted plan.
__device__ __forceinline__ int clamp_idx(int i, int n) { return min(max(i, 0), n - 1); }

// XCD-aware remap of a 1-D grid: hardware hands consecutive workgroups to the 8 XCDs in turn,
// each with its own L2.  The logical tiles are cut into chunks of CHUNK consecutive tiles and the
// chunks are dealt to the XCDs in turn, so that the tiles an XCD runs side by side are neighbours
// (they share operands in its L2) while every XCD still gets an even share of the whole range
// (tiles late in the list can carry more work than early ones).  The tail that does not fill a
// chunk per XCD is split evenly.  `n` must be a multiple of 8; the map is a bijection of [0, n).
// The default chunk is one tile per CU of an XCD; a kernel whose tile groups (RASTER_M m-tiles x
// its n-tiles) are larger takes a chunk that keeps more of a group on one XCD (measured per
// kernel on the fine-grained layer: the half-width down GEMM, 12 n-tiles, 0.394 -> 0.379 ms at
// 96; the dX GEMM, 6 n-tiles, 0.612 -> 0.601 ms at 64; the others best at 32).
constexpr int XCD_CHUNK = 32;
template <int CHUNK = XCD_CHUNK>
__host__ __device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n >> 3;        // workgroups per XCD
  const int xcd = bid & 7, j = bid >> 3;
  const int full = per / CHUNK;  // whole chunks per XCD
  if (j < full * CHUNK) return ((j / CHUNK) * 8 + xcd) * CHUNK + j % CHUNK;
  const int rem = per - full * CHUNK;
  return full * 8 * CHUNK + xcd * rem + (j - full * CHUNK);
}
}  // namespace moe

// MFMA GEMM engine for gfx950, shared by every expert and router GEMM of the layer.
//
// C[m][n] = sum_k A(m,k) B(k,n), fp32 accumulation in MFMA accumulators.
//   * workgroup = 256 threads = 4 waves in a 2 (M) x 2 (N) grid; block tile 256 x 256;
//   * each wave owns 128 x 128 = 4 x 4 MFMA 32x32 blocks (the accumulators live in AGPRs); per
//     MFMA k-step a wave reads 8 fragments for 16 MFMAs, which keeps the LDS traffic of fragment
//     reads plus DMA writes within the LDS bandwidth at full MFMA rate
//     (bf16: v_mfma_f32_32x32x16_bf16; fp32: v_mfma_f32_32x32x2_f32);
//   * LDS = four 36 KiB buffers.
//
// bf16 path — a four-deep ring of K stages (32 k per stage) filled by direct global->LDS loads
// (global_load_lds_dwordx4: each lane moves 16 bytes straight into LDS, no registers), issued
// three stages ahead of the MFMAs.  This is the gfx950 form of the SonicMoE page's asynchronous
// "Gather+Load -> GEMM" (its kernels overlap IO with MMA through cp.async; section "Gather
// 与加载融合"): the gathered row pointers feed the DMA directly.  One wave instruction fills
// 1 KiB of contiguous LDS (lane l -> byte 16 l), so tiles are unpadded and XOR-swizzled:
//   * K-major operand (rows with contiguous K: activations, [out][in] weights): [256][64 B];
//     16-byte chunk c of row r sits at slot c ^ ((r >> 2) & 3).  An MFMA fragment is one
//     ds_read_b128 per lane; 16 consecutive rows hit 16 distinct bank groups.
//   * MN-major operand (rows indexed by k, contiguous along M or N: dY / X / dH rows feeding a
//     weight gradient, or weights read transposed): [32 k][256 mn = 512 B]; chunk c of k-row k
//     sits at slot c ^ (4 (k & 3)), and fragments are read with the transposing LDS load
//     ds_read_b64_tr_b16.  Within a 16-lane group, lane i supplies 4 consecutive 16-bit
//     elements and lane j receives element j%4 of lanes j/4, j/4+4, j/4+8, j/4+12 (verified on
//     gfx950): lane i points at k-row i/4, column 4 (i%4), so lane j receives 4 consecutive k of
//     column j; two such loads make the 8 k-values of an MFMA fragment.
//   Invalid rows / columns are loaded from a zero page, so padding contributes zeros.
//   Waits: each thread issues 8 DMA instructions per stage, in order; before a stage is read it
//   waits until at most 8 * (stages issued after it) are outstanding, then a plain s_barrier (no
//   fence) publishes every wave's DMA writes.  Each ring slot is its own __shared__ array and the
//   loop is unrolled by the ring depth, so the compiler can tell that reading one slot does not
//   conflict with the DMAs still in flight into the others.  Fragment reads are double-buffered
//   in registers so that LDS latency hides behind the previous k-step's MFMAs.
//
// Two further layouts of the same bf16 ring share the wave code: the eight-wave engine (512
// threads, 128 x 64 per wave, two waves per SIMD) and the half-width engine (256 x 128 tiles of
// four such waves, a three-slot ring, two workgroups per CU); see their sections below.
//
// FP8 operands (OCP E4M3 or E5M2) go through the four-wave and half-width rings with one-byte
// elements: a stage's 64 bytes per row are one k-step of v_mfma_scale_f32_32x32x64_f8f6f4, with
// the block scales either held at 1.0 (per-row scales, applied in the epilogue) or loaded beside
// the codes, one E8M0 byte per 32 elements (block-scaled); see the FP8 sections below.
//
// fp32 path (small fp32 layers only) — register-staged double buffer: stage j uses buffers
// 2j (A) and 2j+1 (B) as [256][128 B + 16 B pad]; MN-major fp32 operands are transposed in
// registers while staged.
//
// Accumulator layout (32x32 MFMA, verified on gfx950): register v of lane l holds
//   row (v / 4) * 8 + (l / 32) * 4 + (v % 4), column l % 32.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int GEMM_THREADS = 256;
constexpr int LDS_BUF = 36864;              // bytes per LDS buffer (four per workgroup)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void gmem_void;

// Read-only int32 at base[i] through the scalar cache (i made wave-uniform): used for gathered row
// indices inside the DMA loop, where a vector load would be counted by vmcnt and force the wait
// on every outstanding DMA.
__device__ __forceinline__ int sload_i32(const int32_t* base, int i) {
  typedef const __attribute__((address_space(4))) int32_t cint;
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int u = __builtin_amdgcn_readfirstlane(i);
  return *((cint*)(((uint64_t)hi << 32) | lo) + u);
}

// Zero-filled global memory that invalid operand rows are loaded from.
static __device__ __attribute__((aligned(1024))) char g_zero_page[1024];

struct LdsBufs {
  char* b[4];
};

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static constexpr int BK = 32;                  // k per stage (DMA ring)
  static constexpr int STEPS = BK / 16;
  typedef bf16x8 frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static constexpr int BK = 32;                  // 128 bytes per row per stage
  static constexpr int STEPS = BK / 2;
  typedef float frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

struct WaveAcc {
  f32x16 c[4][4];
};

__device__ __forceinline__ void zero_acc(WaveAcc& acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
}

// ===============================================================================================
// bf16: DMA ring
// ===============================================================================================
constexpr int DMA_B_OFF = 16384;            // B tile offset inside a ring slot (A tile at 0)

// s_waitcnt with only vmcnt <= N (vmcnt is 6 bits: low 4 in [3:0], high 2 in [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void dma16(const void* g, char* lds_uniform) {
  __builtin_amdgcn_global_load_lds((gmem_void*)g, (lds_void*)lds_uniform, 16, 0, 0);
}

// K-major operand: tile row i of the stage <- 64 bytes of row_ptr(i) at K offset 64 s.  Wave w
// instruction q fills rows R0 = (4 q + w) * 16 .. R0 + 15; lane l takes row R0 + l/4 and the
// chunk that lands in its slot: (l & 3) ^ (l >> 4).  row_ptr returns null for an invalid row.
struct KDma {
  const char* g[4];
  int step[4];
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const char* p = row_ptr((4 * q + w) * 16 + (lane >> 2));
      g[q] = p ? p + chunk * 16 : g_zero_page + chunk * 16;
      step[q] = p ? 64 : 0;
    }
  }
  int ps[4];  // stage of the last prepare_q(q)
  __device__ void fetch(int) {}
  __device__ void prepare_q(int s, int q) { ps[q] = s; }
  __device__ void issue_q(int q, char* dst) const {
    const int w = threadIdx.x >> 6;
    dma16(g[q] + (int64_t)ps[q] * step[q], dst + (4 * q + w) * 1024);
  }
  __device__ static bf16x8 frag(const char* t, int row0, int s) {
    const int lane = threadIdx.x & 63;
    const int r = row0 + (lane & 31);
    const int slot = (s * 2 + (lane >> 5)) ^ ((r >> 2) & 3);
    return *reinterpret_cast<const bf16x8*>(t + r * 64 + slot * 16);
  }
};

// MN-major operand: stage k-rows 32 s .. 32 s + 31.  Row k of the operand lives at
// kptr(kidx(k)): kidx maps k to a (uniform) row id, either k itself or a gathered token id read
// with a scalar load, and kptr turns the row id into the global address of element (mn_base, k).
// Both are only ever called with k clamped into [0, klim) (so a gathered index is always read in
// bounds); rows k >= klim load zeros.  Wave w instruction q fills k-rows K0 = (4 q + w) * 2 and
// K0 + 1: lanes 0-31 the first, 32-63 the second; lane slot l % 32 holds chunk
// (l % 32) ^ (4 (k & 3)).
//
// fetch(s) reads the row ids of stage s, prepare_q(s, q) turns them into this lane's source for
// instruction q and issue_q(q, dst) starts it; the main loop calls fetch half a ring step before
// the first prepare_q, so that the scalar loads of a gathered operand land behind
// 15 MFMAs and no refill waits for them.  Everything per lane is a select on a scalar lane mask:
// both row addresses sit in scalar registers, and the choice between the row and the zero page is
// one v_cndmask per half (written out, so that the compiler cannot turn it into a branch and push
// the MFMAs behind the address math).
template <class KIdx, class KPtr>
struct MNDma {
  KIdx kidx;
  KPtr kptr;
  int klim;
  uint32_t off[4];      // lane byte offset of its chunk in the row
  uint64_t okmask[4];   // lanes whose columns are inside the operand
  int nid[4][2];        // row ids of the fetched stage: k-rows K0 and K0 + 1 of each instruction
  __device__ MNDma(KIdx fi, KPtr fp, int klim_, int mn_base, int mn_valid)
      : kidx(fi), kptr(fp), klim(klim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = (4 * q + w) * 2 + (lane >> 5);
      const int chunk = (lane & 31) ^ (4 * (k & 3));
      off[q] = chunk * 16;
      okmask[q] = __builtin_amdgcn_ballot_w64(mn_base + chunk * 8 < mn_valid);
    }
  }
  __device__ void fetch(int s) {
    const int w = threadIdx.x >> 6;
    const int lim = __builtin_amdgcn_readfirstlane(klim);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k0 = __builtin_amdgcn_readfirstlane(s * 32 + (4 * q + w) * 2);
      nid[q][0] = kidx(min(k0, lim - 1));
      nid[q][1] = kidx(min(k0 + 1, lim - 1));
    }
  }
  uint64_t src[4];  // per-lane DMA sources of the last prepare_q(q)
  __device__ void prepare_q(int s, int q) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lim = __builtin_amdgcn_readfirstlane(klim);
    const bool hi = lane >= 32;
    const uint64_t zero = reinterpret_cast<uint64_t>(g_zero_page) + (lane & 31) * 16;
    const uint32_t zl = (uint32_t)zero, zh = (uint32_t)(zero >> 32);
    const int k0 = __builtin_amdgcn_readfirstlane(s * 32 + (4 * q + w) * 2);
    const uint64_t p0 = reinterpret_cast<uint64_t>(kptr(nid[q][0]));
    const uint64_t p1 = reinterpret_cast<uint64_t>(kptr(nid[q][1]));
    const uint64_t row = (hi ? p1 : p0) + off[q];
    const uint64_t kmask = (k0 < lim ? 0x00000000FFFFFFFFull : 0ull) | (k0 + 1 < lim ? 0xFFFFFFFF00000000ull : 0ull);
    const uint64_t m = okmask[q] & kmask;
    uint32_t sl = (uint32_t)row, sh = (uint32_t)(row >> 32);
    asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(sl) : "v"(zl), "s"(m));
    asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(sh) : "v"(zh), "s"(m));
    src[q] = ((uint64_t)sh << 32) | sl;
  }
  __device__ void issue_q(int q, char* dst) const {
    const int w = threadIdx.x >> 6;
    dma16(reinterpret_cast<const void*>(src[q]), dst + (4 * q + w) * 1024);
  }
  __device__ static bf16x8 frag(const char* t, int mn0, int s) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, i = lane & 15;
    const int k = s * 16 + (g >> 1) * 8 + (i >> 2);
    const int mn = mn0 + (g & 1) * 16 + 4 * (i & 3);
    const int col = ((mn >> 3) ^ (4 * (k & 3))) * 16 + (mn & 7) * 2;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + k * 512 + col));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + (k + 4) * 512 + col));
    const v4i16 both[2] = {lo, hi};
    bf16x8 r;
    __builtin_memcpy(&r, both, 16);
    return r;
  }
};

// Fragments of one MFMA k-step for this wave: 4 A blocks (its 128 rows) and 4 B blocks.
struct FragSet {
  bf16x8 a[4], b[4];
};

template <class AL, class BL, class BSub>
__device__ __forceinline__ void load_frags(const char* slot, int ks, int wm, BSub bsub, FragSet& F) {
#pragma unroll
  for (int j = 0; j < 4; ++j) F.b[j] = BL::frag(slot + DMA_B_OFF, bsub(j), ks);
#pragma unroll
  for (int i = 0; i < 4; ++i) F.a[i] = AL::frag(slot, wm * 128 + i * 32, ks);
}

// MFMA blocks p = FROM .. TO-1 of one k-step, block p = (i, j) = (p / 4, p % 4).  Block 0 goes
// first on its own: the compiler waits for all outstanding LDS reads before an MFMA that needs
// fragments, so reads issued after it never delay the current k-step.  The B fragment is the
// MFMA's first operand, so each block accumulates the transposed product: a lane holds one tile
// row and runs of four consecutive columns (acc_m / acc_n below).
template <int FROM, int TO>
__device__ __forceinline__ void mma_range(const FragSet& F, WaveAcc& acc) {
#pragma unroll
  for (int p = FROM; p < TO; ++p) acc.c[p >> 2][p & 3] = Mma<bf16>::mma(F.b[p & 3], F.a[p >> 2], acc.c[p >> 2][p & 3]);
}

// Workgroup barrier without a memory fence (the DMA waits are explicit); the empty asm keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The 15 MFMA blocks p = 1..15 of a k-step in four chunks, with one piece of DMA work per
// operand pair before each chunk, fenced so that at most one DMA instruction goes out per four
// MFMAs: a CU takes about 64 bytes per clock of direct-to-LDS loads, and four waves issuing
// back to back would queue behind that and hold up the MFMAs that follow them.
//   half 1 (k-step 0): chunk c issues instruction 2 + c/2 of the previous stage's refill (A for
//     even c, B for odd c) and prepares instruction c of the next refill stage r, once the
//     previous source of that instruction has gone out;
//   half 2 (k-step 1): chunk c issues instruction c/2 of stage r (A for even c, B for odd c).
template <class AL, class BL>
__device__ __forceinline__ void mma_half1(const FragSet& F, WaveAcc& acc, AL& la, BL& lb, int r,
                                          char* slot) {
  la.issue_q(2, slot);
  la.prepare_q(r, 0);
  lb.prepare_q(r, 0);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<1, 5>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.issue_q(2, slot + DMA_B_OFF);
  la.prepare_q(r, 1);
  lb.prepare_q(r, 1);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<5, 9>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.issue_q(3, slot);
  la.prepare_q(r, 2);
  lb.prepare_q(r, 2);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<9, 13>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.issue_q(3, slot + DMA_B_OFF);
  la.prepare_q(r, 3);
  lb.prepare_q(r, 3);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<13, 16>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
}
template <class AL, class BL>
__device__ __forceinline__ void mma_half2(const FragSet& F, WaveAcc& acc, const AL& la,
                                          const BL& lb, char* slot) {
  la.issue_q(0, slot);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<1, 5>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.issue_q(0, slot + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<5, 9>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.issue_q(1, slot);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<9, 13>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.issue_q(1, slot + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<13, 16>(F, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// One ring step for stage s (two MFMA k-steps).  Each stage's refill is split in two halves of
// four DMA instructions per wave (q = 0, 1 and q = 2, 3 of both operands), issued in the second
// half of step s - 3 and the first half of step s - 2; the slot is free in both (its previous
// stage was consumed before the barrier of step s - 3).  On entry F0 holds stage s's k-step 0
// fragment reads, issued during the previous step, and the row ids of stage s + 3 have been
// fetched during the previous step.
//   1. first k-step 0 MFMA (waits for F0); read k-step 1 into F1; the other 15 MFMAs with the
//      second half of stage s + 2's refill and the address preparation of stage s + 3;
//   2. wait for stage s + 1 -- the DMA issued after its last instruction is stage s + 2, eight
//      instructions per wave -- and barrier: every wave is now done with stage s - 1, whose slot
//      takes stage s + 3 (past the end: the last stage again, never computed, so the DMA count
//      per step is fixed and the waits stay exact);
//   3. first k-step 1 MFMA (waits for F1); read stage s + 1's k-step 0 into F0 (on the last step
//      this reads a valid slot whose contents go unused) and fetch the row ids of stage s + 4;
//      the other 15 MFMAs with the first half of stage s + 3's refill.
// The DMA issue is unconditional and its address never comes from a pointer select: a DMA under
// a branch makes the compiler's wait tracking fall back to draining everything.  With one wave
// per SIMD nothing else hides a stall, so sched_barrier fences pin this order.
template <class AL, class BL, class BSub>
__device__ __forceinline__ void dma_step_split(AL& la, BL& lb, int s, int nkt, const char* cur,
                                               const char* next, char* half2, char* half1,
                                               FragSet& F0, FragSet& F1, WaveAcc& acc, int wm,
                                               BSub bsub) {
  const int r = min(s + 3, nkt - 1);
  mma_range<0, 1>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<AL, BL>(cur, 1, wm, bsub, F1);
  __builtin_amdgcn_sched_barrier(0);
  mma_half1(F0, acc, la, lb, r, half2);
  wait_vmcnt<8>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  mma_range<0, 1>(F1, acc);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<AL, BL>(next, 0, wm, bsub, F0);
  la.fetch(min(s + 4, nkt - 1));
  lb.fetch(min(s + 4, nkt - 1));
  __builtin_amdgcn_sched_barrier(0);
  mma_half2(F1, acc, la, lb, half1);
}

// One ring step for stage s, burst variant: the whole refill of stage s + 3 goes out in the
// second half of step s, one DMA per MFMA, right after the barrier (three stages of prefetch
// distance, for operands whose loads see long latency: gathered rows, MN-major tiles).
//   1. first k-step 0 MFMA (waits for F0); read k-step 1 into F1 and fetch the row ids of stage
//      s + 3; the other 15 MFMAs;
//   2. wait for stage s + 1 (only stage s + 2, eight DMA instructions per wave, was issued after
//      it) and barrier; stage s - 1's slot takes stage s + 3 (past the end: the last stage
//      again);
//   3. first k-step 1 MFMA (waits for F1 and the ids); read stage s + 1's k-step 0 into F0;
//      prepare and issue the refill, spread over the other 15 MFMAs.
template <class AL, class BL, class BSub>
__device__ __forceinline__ void dma_step_burst(AL& la, BL& lb, int s, int nkt, const char* cur,
                                               const char* next, char* refill, FragSet& F0,
                                               FragSet& F1, WaveAcc& acc, int wm, BSub bsub) {
  const int r = min(s + 3, nkt - 1);
  mma_range<0, 1>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<AL, BL>(cur, 1, wm, bsub, F1);
  la.fetch(r);
  lb.fetch(r);
  __builtin_amdgcn_sched_barrier(0);
  mma_range<1, 16>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<8>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  mma_range<0, 1>(F1, acc);
  __builtin_amdgcn_sched_barrier(0);
  load_frags<AL, BL>(next, 0, wm, bsub, F0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    la.prepare_q(r, q);
    lb.prepare_q(r, q);
    la.issue_q(q, refill);
    lb.issue_q(q, refill + DMA_B_OFF);
  }
  mma_range<1, 16>(F1, acc);
  // spread the refill's address arithmetic and DMA issue between the 15 MFMAs
#pragma unroll
  for (int i = 0; i < 15; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
    __builtin_amdgcn_sched_group_barrier(0x006, 12, 0);  // up to 12 VALU / SALU
    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);   // one DMA
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Issues stages 0, 1 and 2 of a tile into ring slots 0, 1 and 2 (SPLIT: the first half of stage
// 2; step 0 issues the rest).  The slots must be free.  Requires nkt >= 1.
template <bool SPLIT, class AL, class BL>
__device__ __forceinline__ void gemm_prologue_dma(AL& la, BL& lb, int nkt, LdsBufs L) {
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int r = min(i, nkt - 1);
    la.fetch(r);
    lb.fetch(r);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      la.prepare_q(r, q);
      lb.prepare_q(r, q);
    }
#pragma unroll
    for (int q = 0; q < ((SPLIT && i == 2) ? 2 : 4); ++q) {
      la.issue_q(q, L.b[i]);
      lb.issue_q(q, L.b[i] + DMA_B_OFF);
    }
  }
  if constexpr (SPLIT) {
    la.fetch(min(3, nkt - 1));  // ids of the stage step 0 prepares
    lb.fetch(min(3, nkt - 1));
  }
}

// The k-steps of a tile whose prologue has been issued: waits for stage 0 and runs all nkt
// steps, accumulating from zero.  Memory operations issued between the prologue and this call
// (a previous tile's epilogue stores) only make the waits longer: loads complete in order among
// themselves, so "at most N operations outstanding" still implies that every load older than
// the newest N has landed.  Ends with the LDS free.
template <bool SPLIT, class AL, class BL, class BSub>
__device__ __forceinline__ void gemm_body_dma(AL& la, BL& lb, int nkt, WaveAcc& acc, LdsBufs L, int wm,
                                              BSub bsub) {
  zero_acc(acc);
  FragSet F0, F1;
  if constexpr (SPLIT) wait_vmcnt<12>();  // stage 0 has landed: stage 1 (8) and half of stage 2 (4) came after it
  else wait_vmcnt<16>();                  // stage 0 has landed: stages 1 and 2 (16) came after it
  ring_barrier();
  load_frags<AL, BL>(L.b[0], 0, wm, bsub, F0);
  auto step = [&](int st, char* b0, char* b1, char* b2, char* b3) {
    if constexpr (SPLIT) dma_step_split(la, lb, st, nkt, b0, b1, b2, b3, F0, F1, acc, wm, bsub);
    else dma_step_burst(la, lb, st, nkt, b0, b1, b3, F0, F1, acc, wm, bsub);
  };
  int s = 0;
  for (; s + 4 <= nkt; s += 4) {  // full groups: no branches between the steps
    step(s, L.b[0], L.b[1], L.b[2], L.b[3]);
    step(s + 1, L.b[1], L.b[2], L.b[3], L.b[0]);
    step(s + 2, L.b[2], L.b[3], L.b[0], L.b[1]);
    step(s + 3, L.b[3], L.b[0], L.b[1], L.b[2]);
  }
  // 0 to 3 remaining stages; the ring position is again at slot 0
  if (s < nkt) step(s, L.b[0], L.b[1], L.b[2], L.b[3]);
  if (s + 1 < nkt) step(s + 1, L.b[1], L.b[2], L.b[3], L.b[0]);
  if (s + 2 < nkt) step(s + 2, L.b[2], L.b[3], L.b[0], L.b[1]);
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// The bf16 main loop over nkt stages.  SPLIT selects dma_step_split (each refill in two halves,
// one DMA per four MFMAs: for K-major operands with good cache locality) or dma_step_burst.
template <bool SPLIT, class AL, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_dma(AL& la, BL& lb, int nkt, WaveAcc& acc,
                                                  LdsBufs L, int wm, BSub bsub) {
  if (nkt <= 0) {
    zero_acc(acc);
    return;
  }
  gemm_prologue_dma<SPLIT>(la, lb, nkt, L);
  gemm_body_dma<SPLIT>(la, lb, nkt, acc, L, wm, bsub);
}

// ===============================================================================================
// FP8 (OCP E4M3) operands: 1-byte elements through the same DMA ring.  A stage's 64 bytes per
// row are 64 elements, so K-major loading (KDma) is unchanged and a stage is one k-step of 16
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales; per-row scales are applied by the
// epilogue).  A lane's fragment is 32 consecutive k of its row (lane half h: k 32 h .. 32 h + 31);
// A and B use the same placement, which is all a product with unit block scales needs (the
// instruction's own k order differs; the block-scaled path follows it, see frag8_mx).
// ===============================================================================================
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct FragSet8 {
  i32x8 a[4], b[4];
};

__device__ __forceinline__ i32x8 frag8(const char* t, int row0) {
  const int lane = threadIdx.x & 63;
  const int r = row0 + (lane & 31), h = lane >> 5, sw = (r >> 2) & 3;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(t + r * 64 + ((2 * h) ^ sw) * 16);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(t + r * 64 + ((2 * h + 1) ^ sw) * 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

template <class BSub>
__device__ __forceinline__ void load_frags8(const char* slot, int wm, BSub bsub, FragSet8& F) {
#pragma unroll
  for (int j = 0; j < 4; ++j) F.b[j] = frag8(slot + DMA_B_OFF, bsub(j));
#pragma unroll
  for (int i = 0; i < 4; ++i) F.a[i] = frag8(slot, wm * 128 + i * 32);
}

// Blocks p = FROM .. TO-1, block p = (i, j) = (p / 4, p % 4); B first (transposed block, as in
// the bf16 path).  Scale operands 127 = 2^0 in E8M0.
template <int FROM, int TO>
__device__ __forceinline__ void mma8_range(const FragSet8& F, WaveAcc& acc) {
#pragma unroll
  for (int p = FROM; p < TO; ++p)
    acc.c[p >> 2][p & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[p & 3], F.a[p >> 2], acc.c[p >> 2][p & 3],
                                                                           0, 0, 0, 127, 0, 127);
}

// One ring step for stage s (FP8): F0 holds stage s's fragments.  Its first eight blocks go
// first; then the wait for stage s + 1 and the barrier (every wave is done with stage s - 1,
// whose slot takes stage s + 3 -- past the end, the last stage again, so the DMA count per step
// is fixed); then stage s + 1's fragments are read into F1 and the refill goes out, one
// instruction per operand between pairs of the last eight blocks.
template <class AL, class BL, class BSub>
__device__ __forceinline__ void dma_step_f8(AL& la, BL& lb, int s, int nkt, const char* next, char* refill,
                                            FragSet8& F0, FragSet8& F1, WaveAcc& acc, int wm, BSub bsub) {
  const int r = min(s + 3, nkt - 1);
  mma8_range<0, 1>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.fetch(r);
  lb.fetch(r);
  mma8_range<1, 8>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<8>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_frags8(next, wm, bsub, F1);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    la.prepare_q(r, q);
    lb.prepare_q(r, q);
    la.issue_q(q, refill);
    lb.issue_q(q, refill + DMA_B_OFF);
    __builtin_amdgcn_sched_barrier(0);
    if (q == 0) mma8_range<8, 10>(F0, acc);
    if (q == 1) mma8_range<10, 12>(F0, acc);
    if (q == 2) mma8_range<12, 14>(F0, acc);
    if (q == 3) mma8_range<14, 16>(F0, acc);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The FP8 main loop over nkt stages of 64 elements (prologue as in the bf16 burst schedule).
template <class AL, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_f8(AL& la, BL& lb, int nkt, WaveAcc& acc, LdsBufs L, int wm,
                                                 BSub bsub) {
  zero_acc(acc);
  if (nkt <= 0) return;
  gemm_prologue_dma<false>(la, lb, nkt, L);
  FragSet8 F0, F1;
  wait_vmcnt<16>();  // stage 0 has landed: stages 1 and 2 (16) came after it
  ring_barrier();
  load_frags8(L.b[0], wm, bsub, F0);
  int s = 0;
  for (; s + 4 <= nkt; s += 4) {
    dma_step_f8(la, lb, s, nkt, L.b[1], L.b[3], F0, F1, acc, wm, bsub);
    dma_step_f8(la, lb, s + 1, nkt, L.b[2], L.b[0], F1, F0, acc, wm, bsub);
    dma_step_f8(la, lb, s + 2, nkt, L.b[3], L.b[1], F0, F1, acc, wm, bsub);
    dma_step_f8(la, lb, s + 3, nkt, L.b[0], L.b[2], F1, F0, acc, wm, bsub);
  }
  if (s < nkt) dma_step_f8(la, lb, s, nkt, L.b[1], L.b[3], F0, F1, acc, wm, bsub);
  if (s + 1 < nkt) dma_step_f8(la, lb, s + 1, nkt, L.b[2], L.b[0], F1, F0, acc, wm, bsub);
  if (s + 2 < nkt) dma_step_f8(la, lb, s + 2, nkt, L.b[3], L.b[1], F0, F1, acc, wm, bsub);
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// ===============================================================================================
// fp32: register-staged double buffer
// ===============================================================================================
constexpr int KROW = 128 + 16;              // padded K-major row pitch (bytes)

struct RowLoaderF32 {                       // K-major rows: thread owns rows tid/8 + 32 q
  const char* rp[8];
  u32x4 v[8];
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
#pragma unroll
    for (int q = 0; q < 8; ++q) rp[q] = row_ptr((threadIdx.x >> 3) + 32 * q);
  }
  __device__ void load(int kt) {
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (rp[q]) v[q] = ld16(rp[q] + (int64_t)kt * 128 + chunk * 16);
      else v[q] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ void store(char* lds) const {
    const int chunk = threadIdx.x & 7;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      *reinterpret_cast<u32x4*>(lds + ((threadIdx.x >> 3) + 32 * q) * KROW + chunk * 16) = v[q];
  }
  __device__ static float frag(const char* lds, int row0, int s) {
    const int lane = threadIdx.x & 63;
    return *reinterpret_cast<const float*>(lds + (row0 + (lane & 31)) * KROW + s * 8 + (lane >> 5) * 4);
  }
};

// MN-major fp32 operand, transposed in registers into the K-major layout: thread owns two 4 (k)
// x 4 (mn) blocks, mn = 4 (tid % 64), k = 4 (tid / 64) and 4 (tid / 64 + 4).  kbase / klim as
// for MNDma.
template <class KBase>
struct ColLoaderF32 {
  KBase kbase;
  int klim;
  u32x4 v[2][4];
  bool ok;
  __device__ ColLoaderF32(KBase f, int klim_, int mn_base, int mn_valid) : kbase(f), klim(klim_) {
    ok = mn_base + (int)(threadIdx.x & 63) * 4 < mn_valid;
  }
  __device__ void load(int kt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k0 = kt * 32 + ((int)(threadIdx.x >> 6) + 4 * h) * 4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (ok && k0 + kk < klim) v[h][kk] = ld16(kbase(k0 + kk) + (threadIdx.x & 63) * 16);
        else v[h][kk] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  __device__ void store(char* lds) const {
    const int mn0 = (threadIdx.x & 63) * 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int kq = (threadIdx.x >> 6) + 4 * h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u32x4 o{v[h][0][e], v[h][1][e], v[h][2][e], v[h][3][e]};
        *reinterpret_cast<u32x4*>(lds + (mn0 + e) * KROW + kq * 16) = o;
      }
    }
  }
  __device__ static float frag(const char* lds, int row0, int s) { return RowLoaderF32::frag(lds, row0, s); }
};

template <class LA, class LB, class BSub>
__device__ __forceinline__ void gemm_mainloop_reg(LA& la, LB& lb, int nkt, WaveAcc& acc, LdsBufs L,
                                                  int wm, BSub bsub) {
  zero_acc(acc);
  if (nkt <= 0) return;
  la.load(0);
  lb.load(0);
  la.store(L.b[0]);
  lb.store(L.b[1]);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const char* As = (kt & 1) ? L.b[2] : L.b[0];
    const char* Bs = (kt & 1) ? L.b[3] : L.b[1];
    const bool more = kt + 1 < nkt;
    if (more) {
      la.load(kt + 1);
      lb.load(kt + 1);
    }
#pragma unroll
    for (int s = 0; s < Mma<float>::STEPS; ++s) {
      float a[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = LB::frag(Bs, bsub(j), s);
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = LA::frag(As, wm * 128 + i * 32, s);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc.c[i][j] = Mma<float>::mma(b[j], a[i], acc.c[i][j]);
    }
    if (more) {
      la.store((kt & 1) ? L.b[0] : L.b[2]);
      lb.store((kt & 1) ? L.b[1] : L.b[3]);
    }
    __syncthreads();
  }
}

// ===============================================================================================
// Operand builders: one call site per operand kind works for both element types.
//   k_rows<T>(row_ptr)                  K-major rows (row_ptr(i) -> row start or null)
//   mn_rows<T>(kbase, klim, mn_base, mn_valid)
//                                       MN-major rows (kbase(k) -> element (mn_base, k), k < klim)
// and the main loop dispatch gemm_mainloop<T>(la, lb, nkt, acc, L, wm, bsub).
// ===============================================================================================
template <typename T> struct KRowsOf;
template <> struct KRowsOf<bf16> { typedef KDma type; };
template <> struct KRowsOf<float> { typedef RowLoaderF32 type; };

template <typename T, class RowPtr>
__device__ __forceinline__ typename KRowsOf<T>::type k_rows(RowPtr row_ptr) {
  typename KRowsOf<T>::type l;
  l.init(row_ptr);
  return l;
}

struct KIdentity {
  __device__ int operator()(int k) const { return k; }
};

template <typename T, class KBase>
__device__ __forceinline__ auto mn_rows(KBase kbase, int klim, int mn_base, int mn_valid) {
  if constexpr (sizeof(T) == 2) return MNDma<KIdentity, KBase>(KIdentity{}, kbase, klim, mn_base, mn_valid);
  else return ColLoaderF32<KBase>(kbase, klim, mn_base, mn_valid);
}

// MN-major rows through an index: row k at kptr(kidx(k)), kidx returning a uniform row id.
template <typename T, class KIdx, class KPtr>
__device__ __forceinline__ auto mn_rows_idx(KIdx kidx, KPtr kptr, int klim, int mn_base, int mn_valid) {
  if constexpr (sizeof(T) == 2) {
    return MNDma<KIdx, KPtr>(kidx, kptr, klim, mn_base, mn_valid);
  } else {
    auto kbase = [=](int k) { return kptr(kidx(k)); };
    return ColLoaderF32<decltype(kbase)>(kbase, klim, mn_base, mn_valid);
  }
}

// SPLIT: see gemm_mainloop_dma (bf16 only; the fp32 path has one schedule).
template <typename T, bool SPLIT = false, class LA, class LB, class BSub>
__device__ __forceinline__ void gemm_mainloop(LA& la, LB& lb, int nkt, WaveAcc& acc, LdsBufs L, int wm,
                                              BSub bsub) {
  if constexpr (sizeof(T) == 2) gemm_mainloop_dma<SPLIT>(la, lb, nkt, acc, L, wm, bsub);
  else gemm_mainloop_reg(la, lb, nkt, acc, L, wm, bsub);
}

// K stages for a K extent of `k` elements.
template <typename T> __host__ __device__ constexpr int stage_k() { return Mma<T>::BK; }

// First tile column (within the 256-wide tile) of N block j of wave column wn; the block covers
// 32 columns from there (lane l's B fragment is column + l % 32):
//   plain:  wn * 128 + j * 32
//   halved: (j / 2) * 128 + wn * 64 + (j % 2) * 32   (each 128-column half of the tile holds two
//           of the wave's blocks: used where the tile's halves are gate and up, or where the
//           epilogue works one half at a time)
__device__ __forceinline__ int bsub_plain(int wn, int j) { return wn * 128 + j * 32; }
__device__ __forceinline__ int bsub_halved(int wn, int j) { return (j >> 1) * 128 + wn * 64 + (j & 1) * 32; }

// Accumulator placement (the MFMAs compute the transposed block): register v of block (i, j)
// of wave (wm, wn) holds tile row acc_m(wm, i) and column bsub(wn, j) + acc_n(v); registers
// 4q .. 4q + 3 are four consecutive columns of the same row.
__device__ __forceinline__ int acc_m(int wm, int i) { return wm * 128 + i * 32 + (threadIdx.x & 31); }
__device__ __forceinline__ int acc_n(int v) { return (v >> 2) * 8 + ((threadIdx.x >> 5) & 1) * 4 + (v & 3); }

// ---------------------------------------------------------------------------------------------
// Epilogue through LDS for 2-byte outputs.  Tile row r lives in buffer r / 64 at row r % 64 of a
// [64][256 bf16 + 16 B] staging array.  epi_stage_bf16 writes val(i, j, v) at (acc_m, col(j) +
// acc_n(v)), four consecutive columns per 8-byte LDS write (col(j) < 0 skips block j);
// epi_store_bf16 stores rows < mrows and columns < ncols_valid with 16-byte writes through
// row_ptr(r) (null skips).  Requires the LDS to be free.
// ---------------------------------------------------------------------------------------------
constexpr int EPI_ROW = 256 * 2 + 16;
static_assert(64 * EPI_ROW <= LDS_BUF, "staging rows per buffer");

__device__ __forceinline__ char* epi_buf(LdsBufs L, int r) {
  return r < 128 ? (r < 64 ? L.b[0] : L.b[1]) : (r < 192 ? L.b[2] : L.b[3]);
}
__device__ __forceinline__ char* epi_row(LdsBufs L, int r) { return epi_buf(L, r) + (r & 63) * EPI_ROW; }

template <class Col, class Val>
__device__ __forceinline__ void epi_stage_bf16(LdsBufs L, int wm, Col col, Val val) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = col(j);
    if (c < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      char* row = epi_row(L, acc_m(wm, i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 pk = {pack_bf16x2(val(i, j, 4 * q), val(i, j, 4 * q + 1)),
                          pack_bf16x2(val(i, j, 4 * q + 2), val(i, j, 4 * q + 3))};
        *reinterpret_cast<u32x2*>(row + (c + acc_n(4 * q)) * 2) = pk;
      }
    }
  }
}

// Stores the staged rows 0..mrows-1, columns col0 .. col0 + ncols_valid - 1 (ncols = 128 or 256),
// as 16-byte chunks: eight LDS reads per thread are issued before their eight stores, so the
// stores do not each wait out an LDS read.  Streaming (non-temporal) stores: the results are
// read back by a later kernel, not by this one.
template <int NTHR = GEMM_THREADS, class RowPtr>
__device__ __forceinline__ void epi_store_rows(LdsBufs L, int col0, RowPtr row_ptr, int mrows, int ncols,
                                               int ncols_valid) {
  const int cpr = ncols / 8;  // 16-byte chunks per row
  const int total = 256 * cpr;
  constexpr int BATCH = 8;
  for (int c0 = threadIdx.x; c0 < total; c0 += BATCH * NTHR) {
    u32x4 v[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = c0 + b * NTHR;
      const int r = c / cpr, ch = c % cpr;
      if (c < total) v[b] = *reinterpret_cast<const u32x4*>(epi_row(L, r) + col0 * 2 + ch * 16);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int c = c0 + b * NTHR;
      const int r = c / cpr, ch = c % cpr;
      if (c >= total || r >= mrows || ch * 8 >= ncols_valid) continue;
      bf16* p = row_ptr(r);
      if (p) st16_nt(p + ch * 8, v[b]);
    }
  }
}

__device__ __forceinline__ void epi_store_bf16(LdsBufs L, int col0, bf16* out, int64_t ld, int mrows,
                                               int ncols, int ncols_valid) {
  epi_store_rows(L, col0, [&](int r) { return out + (int64_t)r * ld; }, mrows, ncols, ncols_valid);
}

// Direct element stores of a wave's accumulators (the fp32 layers' epilogue): row_ptr(m) is tile
// row m's output at the tile's first column (plain block layout); rows >= mrows and columns >=
// valid are skipped.
template <class RowPtr>
__device__ __forceinline__ void epi_store_direct(int wm, int wn, const WaveAcc& acc, int valid, int mrows,
                                                 RowPtr row_ptr) {
  using T = typename std::remove_pointer<decltype(row_ptr(0))>::type;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = acc_m(wm, i);
    if (m >= mrows) continue;
    T* out = row_ptr(m);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int c = bsub_plain(wn, j) + acc_n(v);
        if (c < valid) out[c] = from_f32<T>(acc.c[i][j][v]);
      }
  }
}

// ===============================================================================================
// Eight waves per workgroup (two per SIMD), for the bf16 GEMMs with an MN-major operand (dX,
// dAct and the weight gradients).  The tile is still 256 x 256 with the same four-slot DMA ring
// and LDS layouts, but each wave computes 128 x 64 (wave row wm = wave / 4, wave column wn =
// wave % 4; 128 accumulator registers), so two waves share a SIMD and one issues MFMAs while the
// other waits out a DMA issue or its address arithmetic.  Each wave issues two DMA instructions
// per operand and stage (instruction q fills row / k-row block 8 q + wave).  Measured: the same
// bits as the four-wave engine, 10% less time on the dX GEMM; a K-major-only GEMM gains less
// (4% on gate/up), because each wave now reads 0.75 instead of 0.5 KB of fragments per MFMA.
// ===============================================================================================
constexpr int GEMM8_THREADS = 512;

// K-major operand (layout as KDma).
struct KDmaW8 {
  const char* g[2];
  int step[2];
  int ps[2];
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const char* p = row_ptr((8 * q + w) * 16 + (lane >> 2));
      g[q] = p ? p + chunk * 16 : g_zero_page + chunk * 16;
      step[q] = p ? 64 : 0;
    }
  }
  template <int P>
  __device__ void fetch(int) {}
  template <int P>
  __device__ void prepare_q(int s, int q) { ps[q] = s; }
  __device__ void issue_q(int q, char* dst) const {
    const int w = threadIdx.x >> 6;
    dma16(g[q] + (int64_t)ps[q] * step[q], dst + (8 * q + w) * 1024);
  }
  __device__ static bf16x8 frag(const char* t, int row0, int s) { return KDma::frag(t, row0, s); }
};

// MN-major operand (layout as MNDma).  The row ids of a stage are fetched into one of two
// buffers by the stage's parity P, so that the ids of the next stage can be read while the
// current one's second half is still to be prepared.
template <class KIdx, class KPtr>
struct MNDmaW8 {
  KIdx kidx;
  KPtr kptr;
  int klim;
  uint32_t off[2];
  uint64_t okmask[2];
  int nid[2][2][2];  // [parity][instruction][k-row K0, K0 + 1]
  uint64_t src[2];
  __device__ MNDmaW8(KIdx fi, KPtr fp, int klim_, int mn_base, int mn_valid) : kidx(fi), kptr(fp), klim(klim_) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k = (8 * q + w) * 2 + (lane >> 5);
      const int chunk = (lane & 31) ^ (4 * (k & 3));
      off[q] = chunk * 16;
      okmask[q] = __builtin_amdgcn_ballot_w64(mn_base + chunk * 8 < mn_valid);
    }
  }
  template <int P>
  __device__ void fetch(int s) {
    const int w = threadIdx.x >> 6;
    const int lim = __builtin_amdgcn_readfirstlane(klim);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int k0 = __builtin_amdgcn_readfirstlane(s * 32 + (8 * q + w) * 2);
      nid[P][q][0] = kidx(min(k0, lim - 1));
      nid[P][q][1] = kidx(min(k0 + 1, lim - 1));
    }
  }
  template <int P>
  __device__ void prepare_q(int s, int q) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lim = __builtin_amdgcn_readfirstlane(klim);
    const bool hi = lane >= 32;
    const uint64_t zero = reinterpret_cast<uint64_t>(g_zero_page) + (lane & 31) * 16;
    const uint32_t zl = (uint32_t)zero, zh = (uint32_t)(zero >> 32);
    const int k0 = __builtin_amdgcn_readfirstlane(s * 32 + (8 * q + w) * 2);
    const uint64_t p0 = reinterpret_cast<uint64_t>(kptr(nid[P][q][0]));
    const uint64_t p1 = reinterpret_cast<uint64_t>(kptr(nid[P][q][1]));
    const uint64_t row = (hi ? p1 : p0) + off[q];
    const uint64_t kmask = (k0 < lim ? 0x00000000FFFFFFFFull : 0ull) | (k0 + 1 < lim ? 0xFFFFFFFF00000000ull : 0ull);
    const uint64_t m = okmask[q] & kmask;
    uint32_t sl = (uint32_t)row, sh = (uint32_t)(row >> 32);
    asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(sl) : "v"(zl), "s"(m));
    asm("v_cndmask_b32_e64 %0, %1, %0, %2" : "+v"(sh) : "v"(zh), "s"(m));
    src[q] = ((uint64_t)sh << 32) | sl;
  }
  __device__ void issue_q(int q, char* dst) const {
    const int w = threadIdx.x >> 6;
    dma16(reinterpret_cast<const void*>(src[q]), dst + (8 * q + w) * 1024);
  }
  __device__ static bf16x8 frag(const char* t, int mn0, int s) { return MNDma<KIdx, KPtr>::frag(t, mn0, s); }
};

template <class KPtr>
__device__ __forceinline__ auto mn_rows_w8(KPtr kptr, int klim, int mn_base, int mn_valid) {
  return MNDmaW8<KIdentity, KPtr>(KIdentity{}, kptr, klim, mn_base, mn_valid);
}
template <class KIdx, class KPtr>
__device__ __forceinline__ auto mn_rows_idx_w8(KIdx kidx, KPtr kptr, int klim, int mn_base, int mn_valid) {
  return MNDmaW8<KIdx, KPtr>(kidx, kptr, klim, mn_base, mn_valid);
}

// A wave's accumulators: 4 row blocks x 2 column blocks of 32 x 32 (transposed blocks, as in
// WaveAcc: acc_m(wm, i) rows, column block j at bsub(j) + acc_n(v)).
struct AccW8 {
  f32x16 c[4][2];
};
struct FragW8 {
  bf16x8 a[4], b[2];
};

template <class AL, class BL, class BSub>
__device__ __forceinline__ void load_frags_w8(const char* slot, int ks, int wm, BSub bsub, FragW8& F) {
#pragma unroll
  for (int j = 0; j < 2; ++j) F.b[j] = BL::frag(slot + DMA_B_OFF, bsub(j), ks);
#pragma unroll
  for (int i = 0; i < 4; ++i) F.a[i] = AL::frag(slot, wm * 128 + i * 32, ks);
}

template <int FROM, int TO>
__device__ __forceinline__ void mma_range_w8(const FragW8& F, AccW8& acc) {
#pragma unroll
  for (int p = FROM; p < TO; ++p)
    acc.c[p >> 1][p & 1] = Mma<bf16>::mma(F.b[p & 1], F.a[p >> 1], acc.c[p >> 1][p & 1]);
}

// One ring step for stage s (P = s & 1).  A stage's refill is split in two: instruction q = 0 of
// both operands goes out in the second half of step s - 3 (into the slot stage s - 4 left, free
// since that step's barrier) and q = 1 in the first half of step s - 2.
//   1. first MFMA of k-step 0; read k-step 1's fragments; fetch the row ids of stage s + 3;
//      issue q = 1 of stage s + 2 beside the other 7 MFMAs;
//   2. wait for stage s + 1 (only the four instructions of stage s + 2 came after it) and
//      barrier;
//   3. first MFMA of k-step 1; read stage s + 1's k-step 0 fragments; issue q = 0 of stage s + 3
//      beside the other 7 MFMAs.
// Stages past the end repeat the last one, so the count of DMA instructions per step, and with
// it every wait, stays fixed.
// MMA = false: the same DMA issue, waits and barriers with no fragment reads and no MFMAs, for a
// wave whose 128 tile rows are all past the valid ones (see gemm_mainloop_w8_rows).
template <int P, bool MMA, class AL, class BL, class BSub>
__device__ __forceinline__ void dma_step_w8(AL& la, BL& lb, int s, int nkt, const char* cur, const char* next,
                                            char* half2, char* refill, FragW8& F0, FragW8& F1, AccW8& acc, int wm,
                                            BSub bsub) {
  const int r2 = min(s + 2, nkt - 1), r3 = min(s + 3, nkt - 1);
  if constexpr (MMA) mma_range_w8<0, 1>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MMA) load_frags_w8<AL, BL>(cur, 1, wm, bsub, F1);
  la.template fetch<P ^ 1>(r3);
  lb.template fetch<P ^ 1>(r3);
  __builtin_amdgcn_sched_barrier(0);
  la.template prepare_q<P>(r2, 1);
  la.issue_q(1, half2);
  if constexpr (MMA) mma_range_w8<1, 4>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.template prepare_q<P>(r2, 1);
  lb.issue_q(1, half2 + DMA_B_OFF);
  if constexpr (MMA) mma_range_w8<4, 8>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<4>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MMA) mma_range_w8<0, 1>(F1, acc);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MMA) load_frags_w8<AL, BL>(next, 0, wm, bsub, F0);
  __builtin_amdgcn_sched_barrier(0);
  la.template prepare_q<P ^ 1>(r3, 0);
  la.issue_q(0, refill);
  if constexpr (MMA) mma_range_w8<1, 4>(F1, acc);
  __builtin_amdgcn_sched_barrier(0);
  lb.template prepare_q<P ^ 1>(r3, 0);
  lb.issue_q(0, refill + DMA_B_OFF);
  if constexpr (MMA) mma_range_w8<4, 8>(F1, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// The eight-wave main loop over nkt stages (accumulating from zero; ends with the LDS free).
template <bool MMA = true, class AL, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_w8(AL& la, BL& lb, int nkt, AccW8& acc, LdsBufs L, int wm, BSub bsub) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nkt <= 0) return;
  // stages 0 and 1 whole, stage 2's instruction 0 (step 0 issues its instruction 1)
  la.template fetch<0>(0);
  lb.template fetch<0>(0);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    la.template prepare_q<0>(0, q);
    lb.template prepare_q<0>(0, q);
    la.issue_q(q, L.b[0]);
    lb.issue_q(q, L.b[0] + DMA_B_OFF);
  }
  const int r1 = min(1, nkt - 1), r2 = min(2, nkt - 1);
  la.template fetch<1>(r1);
  lb.template fetch<1>(r1);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    la.template prepare_q<1>(r1, q);
    lb.template prepare_q<1>(r1, q);
    la.issue_q(q, L.b[1]);
    lb.issue_q(q, L.b[1] + DMA_B_OFF);
  }
  la.template fetch<0>(r2);
  lb.template fetch<0>(r2);
  la.template prepare_q<0>(r2, 0);
  lb.template prepare_q<0>(r2, 0);
  la.issue_q(0, L.b[2]);
  lb.issue_q(0, L.b[2] + DMA_B_OFF);
  wait_vmcnt<6>();  // stage 0 has landed: stage 1 (4) and half of stage 2 (2) came after it
  ring_barrier();
  FragW8 F0, F1;
  if constexpr (MMA) load_frags_w8<AL, BL>(L.b[0], 0, wm, bsub, F0);
  int s = 0;
  for (; s + 4 <= nkt; s += 4) {
    dma_step_w8<0, MMA>(la, lb, s, nkt, L.b[0], L.b[1], L.b[2], L.b[3], F0, F1, acc, wm, bsub);
    dma_step_w8<1, MMA>(la, lb, s + 1, nkt, L.b[1], L.b[2], L.b[3], L.b[0], F0, F1, acc, wm, bsub);
    dma_step_w8<0, MMA>(la, lb, s + 2, nkt, L.b[2], L.b[3], L.b[0], L.b[1], F0, F1, acc, wm, bsub);
    dma_step_w8<1, MMA>(la, lb, s + 3, nkt, L.b[3], L.b[0], L.b[1], L.b[2], F0, F1, acc, wm, bsub);
  }
  if (s < nkt) dma_step_w8<0, MMA>(la, lb, s, nkt, L.b[0], L.b[1], L.b[2], L.b[3], F0, F1, acc, wm, bsub);
  if (s + 1 < nkt) dma_step_w8<1, MMA>(la, lb, s + 1, nkt, L.b[1], L.b[2], L.b[3], L.b[0], F0, F1, acc, wm, bsub);
  if (s + 2 < nkt) dma_step_w8<0, MMA>(la, lb, s + 2, nkt, L.b[2], L.b[3], L.b[0], L.b[1], F0, F1, acc, wm, bsub);
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// The eight-wave main loop for a tile with `mrows` valid rows: a wave whose 128 rows all lie past
// them (wave row 1 of a tile with at most 128 valid rows, e.g. an expert's last tile after token
// rounding to 128) still issues its share of every stage's DMA and meets every barrier, but reads
// no fragments and issues no MFMAs, so the wave row 0 wave on the same SIMD has the matrix unit
// to itself.  Its accumulators stay zero and its rows are never stored.
template <class AL, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_w8_rows(AL& la, BL& lb, int nkt, AccW8& acc, LdsBufs L, int wm,
                                                      BSub bsub, int mrows) {
  if (wm * 128 < mrows) gemm_mainloop_w8<true>(la, lb, nkt, acc, L, wm, bsub);
  else gemm_mainloop_w8<false>(la, lb, nkt, acc, L, wm, bsub);
}

// Column block j of wave column wn (plain layout): 64 columns per wave column.
__device__ __forceinline__ int bsub_w8(int wn, int j) { return wn * 64 + j * 32; }

// Epilogue staging for the eight-wave layout (rows as epi_stage_bf16).
template <class Col, class Val>
__device__ __forceinline__ void epi_stage_w8(LdsBufs L, int wm, Col col, Val val) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = col(j);
    if (c < 0) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      char* row = epi_row(L, acc_m(wm, i));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 pk = {pack_bf16x2(val(i, j, 4 * q), val(i, j, 4 * q + 1)),
                          pack_bf16x2(val(i, j, 4 * q + 2), val(i, j, 4 * q + 3))};
        *reinterpret_cast<u32x2*>(row + (c + acc_n(4 * q)) * 2) = pk;
      }
    }
  }
}

// ===============================================================================================
// Half-width engine: 256 x 128 output tiles, four waves of 128 x 64 (the eight-wave wave tile)
// and a three-slot ring of 24 KB stages, so that two workgroups fit on a CU (72 KB of LDS and at
// most 256 registers per wave each) and one's prologue and epilogue run beside the other's
// main loop.  For the GEMMs with short K, whose tiles spend much of their time filling the ring
// and draining the output (the down GEMMs, the FP8 gate/up GEMM at small d), and for the router
// GEMM, whose N = E (128 on the fine-grained layer) would leave half of a 256-wide tile empty.
// ===============================================================================================
constexpr int HBN = 128;                  // output columns per tile
// The down GEMMs take this engine up to these n (K): 16 bf16 or 32 fp8 stages per tile.  Measured
// on layers with n = 256 (8 / 4 stages: faster), 2048 (64 bf16 stages: slower; 32 fp8 stages:
// faster) and 14336 (slower in both).
constexpr int DOWN_H_MAX_N = 512;
constexpr int DOWN_H_MAX_N_FP8 = 2048;
constexpr int H_SLOT = 24576;             // A 16 KB (256 rows x 64 B) + B 8 KB (128 rows x 64 B)
constexpr int H_EPI_ROW = HBN * 2 + 16;   // staging row pitch of the epilogue
constexpr int H_EPI_ROWS = H_SLOT / H_EPI_ROW;  // staging rows per slot (90; three slots hold 256)
static_assert(3 * H_EPI_ROWS >= BM, "epilogue staging fits the ring");

// K-major operand of the half-width engine (layout as KDma): wave w instruction q fills tile rows
// (4 q + w) * 16 .. + 15; NQ = 4 for the 256 A rows, 2 for the 128 B rows.
template <int NQ>
struct KDmaH {
  const char* g[NQ];
  int step[NQ];
  template <class RowPtr>
  __device__ void init(RowPtr row_ptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const char* p = row_ptr((4 * q + w) * 16 + (lane >> 2));
      g[q] = p ? p + chunk * 16 : g_zero_page + chunk * 16;
      step[q] = p ? 64 : 0;
    }
  }
  __device__ void issue(int q, int s, char* dst) const {
    const int w = threadIdx.x >> 6;
    dma16(g[q] + (int64_t)s * step[q], dst + (4 * q + w) * 1024);
  }
  __device__ static bf16x8 frag(const char* t, int row0, int s) { return KDma::frag(t, row0, s); }
};

// One ring step: wait for stage s (stage s + 1, six instructions, may still be in flight),
// barrier (every wave is done with the slot stage s - 1 used), refill that slot with stage s + 2
// (stages past the end repeat the last one, so every wait counts the same), and the MFMAs of
// stage s with the six DMA instructions spread between them: bf16, two k-steps of 8 blocks; FP8
// (F8), one k-step of 8 v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales.
struct FragH8 {
  i32x8 a[4], b[2];
};
template <int FROM, int TO>
__device__ __forceinline__ void mma8_range_h(const FragH8& F, AccW8& acc) {
#pragma unroll
  for (int p = FROM; p < TO; ++p)
    acc.c[p >> 1][p & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[p & 1], F.a[p >> 1], acc.c[p >> 1][p & 1],
                                                                           0, 0, 0, 127, 0, 127);
}

template <bool F8, class BL, class BSub>
__device__ __forceinline__ void step_h(const KDmaH<4>& la, const BL& lb, int s, int nkt, const char* cur,
                                       char* refill, AccW8& acc, int wm, BSub bsub) {
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<6>();
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const int r = min(s + 2, nkt - 1);
  if constexpr (F8) {
    FragH8 F;
#pragma unroll
    for (int j = 0; j < 2; ++j) F.b[j] = frag8(cur + DMA_B_OFF, bsub(j));
#pragma unroll
    for (int i = 0; i < 4; ++i) F.a[i] = frag8(cur, wm * 128 + i * 32);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(0, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<0, 1>(F, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(1, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<1, 3>(F, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(2, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<3, 5>(F, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(3, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<5, 6>(F, acc);
    __builtin_amdgcn_sched_barrier(0);
    lb.issue(0, r, refill + DMA_B_OFF);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<6, 7>(F, acc);
    __builtin_amdgcn_sched_barrier(0);
    lb.issue(1, r, refill + DMA_B_OFF);
    __builtin_amdgcn_sched_barrier(0);
    mma8_range_h<7, 8>(F, acc);
  } else {
    FragW8 F0, F1;
    load_frags_w8<KDmaH<4>, BL>(cur, 0, wm, bsub, F0);
    load_frags_w8<KDmaH<4>, BL>(cur, 1, wm, bsub, F1);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(0, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<0, 3>(F0, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(1, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<3, 6>(F0, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(2, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<6, 8>(F0, acc);
    mma_range_w8<0, 1>(F1, acc);
    __builtin_amdgcn_sched_barrier(0);
    la.issue(3, r, refill);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<1, 4>(F1, acc);
    __builtin_amdgcn_sched_barrier(0);
    lb.issue(0, r, refill + DMA_B_OFF);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<4, 6>(F1, acc);
    __builtin_amdgcn_sched_barrier(0);
    lb.issue(1, r, refill + DMA_B_OFF);
    __builtin_amdgcn_sched_barrier(0);
    mma_range_w8<6, 8>(F1, acc);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// The half-width main loop over nkt stages (accumulating from zero; ends with the LDS free); a
// stage is 32 bf16 or (F8) 64 fp8 k-values.
template <bool F8, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_h(const KDmaH<4>& la, const BL& lb, int nkt, AccW8& acc,
                                                char* b0, char* b1, char* b2, int wm, BSub bsub) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nkt <= 0) return;
  const int r1 = min(1, nkt - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) la.issue(q, 0, b0);
#pragma unroll
  for (int q = 0; q < 2; ++q) lb.issue(q, 0, b0 + DMA_B_OFF);
#pragma unroll
  for (int q = 0; q < 4; ++q) la.issue(q, r1, b1);
#pragma unroll
  for (int q = 0; q < 2; ++q) lb.issue(q, r1, b1 + DMA_B_OFF);
  int s = 0;
  for (; s + 3 <= nkt; s += 3) {
    step_h<F8>(la, lb, s, nkt, b0, b2, acc, wm, bsub);
    step_h<F8>(la, lb, s + 1, nkt, b1, b0, acc, wm, bsub);
    step_h<F8>(la, lb, s + 2, nkt, b2, b1, acc, wm, bsub);
  }
  if (s < nkt) {  // nested, so that the compiler sees that the second tail step follows the first
    step_h<F8>(la, lb, s, nkt, b0, b2, acc, wm, bsub);
    if (s + 1 < nkt) step_h<F8>(la, lb, s + 1, nkt, b1, b0, acc, wm, bsub);
  }
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// ---------------------------------------------------------------------------------------------
// Block-scaled FP8 on the half-width engine: E4M3 (FMT 0) or E5M2 (FMT 1) codes with one E8M0
// scale byte per 32 consecutive k of each row, applied by v_mfma_scale_f32_32x32x64_f8f6f4 itself.
// Scales are stored group-major, [K / 128][rows][4 bytes]: a group holds the four blocks of 128
// consecutive k of a row, so stage s (64 k) uses bytes 2 (s & 1) and 2 (s & 1) + 1 of the row's
// word in group s / 2, and the words of consecutive rows are contiguous (a wave loads 64 rows'
// words as 256 contiguous bytes).  Each ring slot gets a 2 KB scale area after its codes:
// A words [256 rows][4 B], then B words [128 rows][4 B] twice (see ScaleDmaH).
// ---------------------------------------------------------------------------------------------
constexpr int H_SLOT_MX = H_SLOT + 2048;
constexpr int MX_SA_OFF = H_SLOT;         // A operand scales in a slot
constexpr int MX_SB_OFF = H_SLOT + 1024;  // B operand scales in a slot

// The block-scaled loop's loaders keep, per lane, a 32-bit byte offset from a wave-uniform base
// (one register per instruction instead of a 64-bit pointer and a step), which keeps the loop
// within the 256 registers of two workgroups per CU.  Rows past the valid ones are given the offset
// of a valid row by the caller: their products land in accumulator rows or columns that are never
// stored, so no zero-page select is needed.
// Codes, K-major (layout as KDma): instruction q fills tile rows (4 q + w) * 16 .. + 15 from
// base[q] + off[q] + 64 s (each instruction's rows lie in one source array, so its base is uniform).
template <int NQ>
struct KDmaHU {
  const char* base[NQ];
  uint32_t off[NQ];
  template <class Base, class RowOff>
  __device__ void init(Base base_of, RowOff row_off) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      base[q] = base_of(q);
      off[q] = row_off((4 * q + w) * 16 + (lane >> 2)) + chunk * 16;
    }
  }
  // the stage index goes through readfirstlane, which the compiler cannot see through, so it
  // forms each address when the instruction issues instead of keeping a 64-bit induction pointer
  // per instruction live across the loop
  __device__ void issue(int q, int s, char* dst) const {
    const int w = threadIdx.x >> 6;
    const uint32_t so = (uint32_t)__builtin_amdgcn_readfirstlane(s) * 64u;
    dma16(base[q] + (off[q] + so), dst + (4 * q + w) * 1024);
  }
};

// Scale words of one operand: wave w loads, for the 64 tile rows (w % NG) * 64 + lane, the word
// of stage s's group, straight into LDS at [row][4 B] (global_load_lds_dword: lane l writes 4
// bytes at the wave's destination + 4 l); the group's plane is `plane` bytes past the previous
// one.  NG = 4 for the 256 A rows; NG = 2 for the 128 B rows, where waves 2 and 3 load the rows
// of waves 0 and 1 again into a second copy, so that every wave issues exactly one instruction
// per operand and stage and the waits stay exact.
template <int NG>
struct ScaleDmaH {
  const char* base;
  int64_t plane;
  uint32_t off;
  template <class Base, class RowOff>
  __device__ void init(Base base_of_wave, int64_t plane_bytes, RowOff row_off) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    base = base_of_wave(w % NG);
    plane = plane_bytes;
    off = row_off((w % NG) * 64 + lane);
  }
  __device__ void issue(int s, char* area) const {
    const int w = threadIdx.x >> 6;
    const int64_t so = (int64_t)__builtin_amdgcn_readfirstlane(s >> 1) * plane;
    __builtin_amdgcn_global_load_lds((gmem_void*)(base + so + off), (lds_void*)(area + w * 256), 4, 0, 0);
  }
};

// Fragment of the block-scaled MFMA (measured on gfx950 with one-hot inputs and distinct scales):
// of the 64 k of a 32x32x64 step, lane l (h = l / 32) holds k 16 h .. 16 h + 15 in its bytes 0-15
// and k 32 + 16 h .. 32 + 16 h + 15 in bytes 16-31; k 0-31 form scale block 0, whose byte comes
// from lane l % 32, and k 32-63 block 1, from lane l % 32 + 32.  So lane h reads 16-byte chunks h
// and 2 + h of the row's 64-byte stage: then block 0 is the stage's bytes 0-31 and block 1 its
// bytes 32-63, the two 32-element blocks the scales were computed on.
__device__ __forceinline__ i32x8 frag8_mx(const char* t, int row0) {
  const int lane = threadIdx.x & 63;
  const int r = row0 + (lane & 31), h = lane >> 5, sw = (r >> 2) & 3;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(t + r * 64 + (h ^ sw) * 16);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(t + r * 64 + ((2 + h) ^ sw) * 16);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// One ring step of the block-scaled loop (as step_h with F8: four A and two B code loads per wave
// and stage).  A scale word covers two stages, so only even stages load scales (one A and one B
// load more: eight instructions, six for odd stages) and an odd stage reads its scale bytes from
// the previous stage's slot `sc`: that slot's refill (an odd stage, so codes only) leaves its
// scale area alone, and the next scale load into it comes three steps later.  ODD = s & 1, known
// at compile time in the unrolled loop, fixes the wait count.
template <int FMT, bool ODD, class BL, class BSub>
__device__ __forceinline__ void step_h_mx(const KDmaHU<4>& la, const BL& lb, const ScaleDmaH<4>& sa,
                                          const ScaleDmaH<2>& sb, int s, int nkt, const char* cur, const char* sc,
                                          char* refill, AccW8& acc, int wm, BSub bsub) {
  constexpr bool refill_scales = !ODD;  // stage s + 2 is even
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<ODD ? 8 : 6>();  // stage s + 1 is in flight
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const int r = min(s + 2, nkt - 1);
  const int lane = threadIdx.x & 63;
  const int byte = 2 * (s & 1) + (lane >> 5);  // the scale this lane supplies: block 2 s + lane / 32
  // the lane's scale bytes, packed: byte i of ka for A block i, byte j of kb for B block j (the
  // MFMA's scale op-select picks the byte)
  FragH8 F;
  uint32_t ka = 0, kb = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    F.b[j] = frag8_mx(cur + DMA_B_OFF, bsub(j));
    kb |= (uint32_t)*reinterpret_cast<const uint8_t*>(sc + MX_SB_OFF + (bsub(j) + (lane & 31)) * 4 + byte) << (8 * j);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F.a[i] = frag8_mx(cur, wm * 128 + i * 32);
    ka |= (uint32_t)*reinterpret_cast<const uint8_t*>(sc + MX_SA_OFF + (wm * 128 + i * 32 + (lane & 31)) * 4 + byte)
          << (8 * i);
  }
  auto mma = [&](auto P) {
    constexpr int p = decltype(P)::value;
    acc.c[p >> 1][p & 1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
        F.b[p & 1], F.a[p >> 1], acc.c[p >> 1][p & 1], FMT, FMT, p & 1, (int)kb, p >> 1, (int)ka);
  };
  __builtin_amdgcn_sched_barrier(0);
  la.issue(0, r, refill);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 0>{});
  __builtin_amdgcn_sched_barrier(0);
  la.issue(1, r, refill);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 1>{});
  __builtin_amdgcn_sched_barrier(0);
  la.issue(2, r, refill);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 2>{});
  __builtin_amdgcn_sched_barrier(0);
  la.issue(3, r, refill);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 3>{});
  __builtin_amdgcn_sched_barrier(0);
  lb.issue(0, r, refill + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 4>{});
  __builtin_amdgcn_sched_barrier(0);
  lb.issue(1, r, refill + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 5>{});
  __builtin_amdgcn_sched_barrier(0);
  if (refill_scales) sa.issue(r, refill + MX_SA_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 6>{});
  __builtin_amdgcn_sched_barrier(0);
  if (refill_scales) sb.issue(r, refill + MX_SB_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma(std::integral_constant<int, 7>{});
  __builtin_amdgcn_sched_barrier(0);
}

// The block-scaled main loop over nkt stages of 64 k (accumulating from zero; ends with the LDS
// free).  The slots are H_SLOT_MX bytes each.
template <int FMT, class BL, class BSub>
__device__ __forceinline__ void gemm_mainloop_h_mx(const KDmaHU<4>& la, const BL& lb, const ScaleDmaH<4>& sa,
                                                   const ScaleDmaH<2>& sb, int nkt, AccW8& acc, char* b0, char* b1,
                                                   char* b2, int wm, BSub bsub) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc.c[i][j][v] = 0.0f;
  if (nkt <= 0) return;
  const int r1 = min(1, nkt - 1);
#pragma unroll
  for (int q = 0; q < 4; ++q) la.issue(q, 0, b0);
#pragma unroll
  for (int q = 0; q < 2; ++q) lb.issue(q, 0, b0 + DMA_B_OFF);
  sa.issue(0, b0 + MX_SA_OFF);
  sb.issue(0, b0 + MX_SB_OFF);
#pragma unroll
  for (int q = 0; q < 4; ++q) la.issue(q, r1, b1);
#pragma unroll
  for (int q = 0; q < 2; ++q) lb.issue(q, r1, b1 + DMA_B_OFF);
  // slots: stage s in b[s % 3]; an odd stage's scales in the previous stage's slot
  int s = 0;
  for (; s + 6 <= nkt; s += 6) {
    step_h_mx<FMT, false>(la, lb, sa, sb, s, nkt, b0, b0, b2, acc, wm, bsub);
    step_h_mx<FMT, true>(la, lb, sa, sb, s + 1, nkt, b1, b0, b0, acc, wm, bsub);
    step_h_mx<FMT, false>(la, lb, sa, sb, s + 2, nkt, b2, b2, b1, acc, wm, bsub);
    step_h_mx<FMT, true>(la, lb, sa, sb, s + 3, nkt, b0, b2, b2, acc, wm, bsub);
    step_h_mx<FMT, false>(la, lb, sa, sb, s + 4, nkt, b1, b1, b0, acc, wm, bsub);
    step_h_mx<FMT, true>(la, lb, sa, sb, s + 5, nkt, b2, b1, b1, acc, wm, bsub);
  }
  if (s < nkt) step_h_mx<FMT, false>(la, lb, sa, sb, s, nkt, b0, b0, b2, acc, wm, bsub);
  if (s + 1 < nkt) step_h_mx<FMT, true>(la, lb, sa, sb, s + 1, nkt, b1, b0, b0, acc, wm, bsub);
  if (s + 2 < nkt) step_h_mx<FMT, false>(la, lb, sa, sb, s + 2, nkt, b2, b2, b1, acc, wm, bsub);
  if (s + 3 < nkt) step_h_mx<FMT, true>(la, lb, sa, sb, s + 3, nkt, b0, b2, b2, acc, wm, bsub);
  if (s + 4 < nkt) step_h_mx<FMT, false>(la, lb, sa, sb, s + 4, nkt, b1, b1, b0, acc, wm, bsub);
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// ---------------------------------------------------------------------------------------------
// Block-scaled FP8 on the four-wave engine (256 x 256 tiles, the ring of gemm_mainloop_f8), for
// long K where the larger tile's operand reuse wins: each slot holds the codes (A 16 KB, B 16 KB)
// and then the A and B scale words ([256 rows][4 B] each).  Per wave and stage: four A and four B
// code loads, and on even stages one A and one B scale load.
// ---------------------------------------------------------------------------------------------
constexpr int F4_SA_OFF = 32768;
constexpr int F4_SB_OFF = 33792;
static_assert(F4_SB_OFF + 1024 <= LDS_BUF, "scale words fit a four-wave slot");

struct FragSet8S {
  i32x8 a[4], b[4];
  uint32_t ra[4], rb[4];  // the lane's scale byte of A block i / B block j, as read
  uint32_t ka, kb;        // the same packed: byte i of ka, byte j of kb
};

// Fragments of stage s from a four-wave slot and its scale bytes from `sslot` (layouts as in
// step_h_mx).  The bytes are packed by pack_scales8s, which the ring step runs after the stage's last MFMAs: packing
// here would make the wave wait for these LDS reads before its next MFMAs.
template <class BSub>
__device__ __forceinline__ void load_frags8s(const char* slot, const char* sslot, int s, int wm, BSub bsub,
                                             FragSet8S& F) {
  const int lane = threadIdx.x & 63;
  const int byte = 2 * (s & 1) + (lane >> 5);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    F.b[j] = frag8_mx(slot + DMA_B_OFF, bsub(j));
    F.rb[j] = *reinterpret_cast<const uint8_t*>(sslot + F4_SB_OFF + (bsub(j) + (lane & 31)) * 4 + byte);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    F.a[i] = frag8_mx(slot, wm * 128 + i * 32);
    F.ra[i] = *reinterpret_cast<const uint8_t*>(sslot + F4_SA_OFF + (wm * 128 + i * 32 + (lane & 31)) * 4 + byte);
  }
}

__device__ __forceinline__ void pack_scales8s(FragSet8S& F) {
  F.ka = F.ra[0] | (F.ra[1] << 8) | (F.ra[2] << 16) | (F.ra[3] << 24);
  F.kb = F.rb[0] | (F.rb[1] << 8) | (F.rb[2] << 16) | (F.rb[3] << 24);
}

// Blocks p = FROM .. TO-1, block p = (i, j) = (p / 4, p % 4), B first as in mma8_range, with the
// blocks' scale bytes selected from the packed words.
template <int FMT, int P>
__device__ __forceinline__ void mma8s_one(const FragSet8S& F, WaveAcc& acc) {
  acc.c[P >> 2][P & 3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
      F.b[P & 3], F.a[P >> 2], acc.c[P >> 2][P & 3], FMT, FMT, P & 3, (int)F.kb, P >> 2, (int)F.ka);
}
template <int FMT, int FROM, int TO>
__device__ __forceinline__ void mma8s_range(const FragSet8S& F, WaveAcc& acc) {
  if constexpr (FROM < TO) {
    mma8s_one<FMT, FROM>(F, acc);
    mma8s_range<FMT, FROM + 1, TO>(F, acc);
  }
}

// One ring step for stage s (as dma_step_f8): the first eight blocks of stage s; the wait for
// stage s + 1 (only stage s + 2 was issued after it) and the barrier; stage s + 1's fragments and
// scales into F1; the refill of stage s + 3 into the slot stage s - 1 used, its instructions
// between pairs of the last eight blocks.  A scale word covers two stages (a group of four
// 32-element blocks), so only even stages load scales (ten instructions per wave, eight for odd
// ones) and an odd stage reads them from the previous stage's slot: that slot is refilled one step
// later, after the barrier that follows every wave's reads.  ODD = s & 1, known at compile time
// in the unrolled loop, fixes each step's wait count.
template <int FMT, bool ODD, class BSub>
__device__ __forceinline__ void dma_step_f8_mx(const KDmaHU<4>& la, const KDmaHU<4>& lb, const ScaleDmaH<4>& sa,
                                               const ScaleDmaH<4>& sb, int s, int nkt, const char* cur,
                                               const char* next, char* refill, FragSet8S& F0, FragSet8S& F1,
                                               WaveAcc& acc, int wm, BSub bsub) {
  constexpr bool refill_scales = ODD;  // stage s + 3 is even
  const int r = min(s + 3, nkt - 1);
  mma8s_range<FMT, 0, 8>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<ODD ? 8 : 10>();  // stage s + 2 (even when s is) is in flight
  ring_barrier();
  __builtin_amdgcn_sched_barrier(0);
  load_frags8s(next, ODD ? next : cur, s + 1, wm, bsub, F1);
  __builtin_amdgcn_sched_barrier(0);
  la.issue(0, r, refill);
  lb.issue(0, r, refill + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma8s_range<FMT, 8, 10>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.issue(1, r, refill);
  lb.issue(1, r, refill + DMA_B_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma8s_range<FMT, 10, 12>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.issue(2, r, refill);
  lb.issue(2, r, refill + DMA_B_OFF);
  if (refill_scales) sa.issue(r, refill + F4_SA_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma8s_range<FMT, 12, 14>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  la.issue(3, r, refill);
  lb.issue(3, r, refill + DMA_B_OFF);
  if (refill_scales) sb.issue(r, refill + F4_SB_OFF);
  __builtin_amdgcn_sched_barrier(0);
  mma8s_range<FMT, 14, 16>(F0, acc);
  __builtin_amdgcn_sched_barrier(0);
  pack_scales8s(F1);
  __builtin_amdgcn_sched_barrier(0);
}

// The four-wave block-scaled main loop over nkt stages of 64 k (stages 0-2 issued first; ends
// with the LDS free).
template <int FMT, class BSub>
__device__ __forceinline__ void gemm_mainloop_f8_mx(const KDmaHU<4>& la, const KDmaHU<4>& lb, const ScaleDmaH<4>& sa,
                                                    const ScaleDmaH<4>& sb, int nkt, WaveAcc& acc, LdsBufs L, int wm,
                                                    BSub bsub) {
  zero_acc(acc);
  if (nkt <= 0) return;
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int r = min(i, nkt - 1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      la.issue(q, r, L.b[i]);
      lb.issue(q, r, L.b[i] + DMA_B_OFF);
    }
    if (i != 1) {
      sa.issue(r, L.b[i] + F4_SA_OFF);
      sb.issue(r, L.b[i] + F4_SB_OFF);
    }
  }
  FragSet8S F0, F1;
  wait_vmcnt<18>();  // stage 0 has landed: stages 1 (8) and 2 (10) came after it
  ring_barrier();
  load_frags8s(L.b[0], L.b[0], 0, wm, bsub, F0);
  pack_scales8s(F0);
  int s = 0;
  for (; s + 4 <= nkt; s += 4) {
    dma_step_f8_mx<FMT, false>(la, lb, sa, sb, s, nkt, L.b[0], L.b[1], L.b[3], F0, F1, acc, wm, bsub);
    dma_step_f8_mx<FMT, true>(la, lb, sa, sb, s + 1, nkt, L.b[1], L.b[2], L.b[0], F1, F0, acc, wm, bsub);
    dma_step_f8_mx<FMT, false>(la, lb, sa, sb, s + 2, nkt, L.b[2], L.b[3], L.b[1], F0, F1, acc, wm, bsub);
    dma_step_f8_mx<FMT, true>(la, lb, sa, sb, s + 3, nkt, L.b[3], L.b[0], L.b[2], F1, F0, acc, wm, bsub);
  }
  if (s < nkt) dma_step_f8_mx<FMT, false>(la, lb, sa, sb, s, nkt, L.b[0], L.b[1], L.b[3], F0, F1, acc, wm, bsub);
  if (s + 1 < nkt) dma_step_f8_mx<FMT, true>(la, lb, sa, sb, s + 1, nkt, L.b[1], L.b[2], L.b[0], F1, F0, acc, wm, bsub);
  if (s + 2 < nkt) dma_step_f8_mx<FMT, false>(la, lb, sa, sb, s + 2, nkt, L.b[2], L.b[3], L.b[1], F0, F1, acc, wm, bsub);
  __syncthreads();  // drains the trailing loads; the LDS is free for the epilogue
}

// Epilogue of a half-width tile: val(i, j, v) of every accumulator staged in bf16, H_EPI_ROWS rows
// to a slot, then stored as 16-byte chunks (rows < mrows, columns < valid) through row_ptr(r).
__device__ __forceinline__ char* epi_row_h(char* b0, char* b1, char* b2, int r) {
  return r < H_EPI_ROWS ? b0 + r * H_EPI_ROW
                        : (r < 2 * H_EPI_ROWS ? b1 + (r - H_EPI_ROWS) * H_EPI_ROW : b2 + (r - 2 * H_EPI_ROWS) * H_EPI_ROW);
}
template <class Val, class BSub, class RowPtr>
__device__ __forceinline__ void epi_h(Val val, char* b0, char* b1, char* b2, int wm, BSub bsub, RowPtr row_ptr,
                                      int mrows, int valid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    char* row = epi_row_h(b0, b1, b2, acc_m(wm, i));
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const u32x2 pk = {pack_bf16x2(val(i, j, 4 * q), val(i, j, 4 * q + 1)),
                          pack_bf16x2(val(i, j, 4 * q + 2), val(i, j, 4 * q + 3))};
        *reinterpret_cast<u32x2*>(row + (bsub(j) + acc_n(4 * q)) * 2) = pk;
      }
  }
  __syncthreads();
#pragma unroll
  for (int b0_ = 0; b0_ < 16; b0_ += 8) {
    u32x4 v[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = threadIdx.x + (b0_ + b) * GEMM_THREADS;
      v[b] = *reinterpret_cast<const u32x4*>(epi_row_h(b0, b1, b2, c >> 4) + (c & 15) * 16);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int c = threadIdx.x + (b0_ + b) * GEMM_THREADS;
      const int r = c >> 4, ch = c & 15;
      if (r < mrows && ch * 8 < valid) st16_nt(row_ptr(r) + ch * 8, v[b]);
    }
  }
}

// Grouped tiles.  The tile table (3 E + 3 ints, written by k_tile_offsets) orders the experts'
// ceil(rows / BM) m-tiles, each with NT n-tiles, in one of two ways.  TAIL_LAST = false: expert by
// expert, table[0..E] being the exclusive scan of the m-tiles per expert.  TAIL_LAST = true: first
// the head tiles, i.e. every m-tile except a last m-tile with 1..BM/2 rows ("light": the
// eight-wave kernels skip the MFMAs of its empty 128-row half), expert by expert (scan in
// table[E + 1 .. 2 E + 1]); then the light tails, table[2 E + 2] of them, of experts
// table[2 E + 3 ..] in ascending order, so that light tiles fill the grid's last round.  Inside an
// expert the tiles run in groups of RASTER_M m-tiles, n-tile outer and m-tile inner, so that the
// workgroups an XCD runs side by side (consecutive `lin`, see xcd_remap) share both their weight
// columns (same n-tile) and their token rows (same group) through that XCD's L2.
struct GroupTile {
  int e, m0, mrows, nt;
};
constexpr int RASTER_M = 8;
// Tile `local` of an MT x NT grid in the grouped order: groups of RASTER_M m-tiles (the last one
// possibly smaller), n-tile outer and m-tile inner inside a group.  Requires local < MT * NT.
__device__ __forceinline__ void raster_tile(int local, int MT, int NT, int& mt, int& nt) {
  const int grp = local / (RASTER_M * NT);
  const int idx = local - grp * RASTER_M * NT;
  const int gm = min(RASTER_M, MT - grp * RASTER_M);
  mt = grp * RASTER_M + idx % gm;
  nt = idx / gm;
}

template <bool TAIL_LAST = false>
__device__ __forceinline__ bool find_group_tile(int lin, int NT, const int32_t* __restrict__ table,
                                                const int32_t* __restrict__ expert_off, int E,
                                                GroupTile& g) {
  const int32_t* scan = TAIL_LAST ? table + E + 1 : table;
  const int heads = scan[E] * NT;
  if (lin >= heads) {
    if (!TAIL_LAST) return false;
    const int k = (lin - heads) / NT;  // light tail k: expert tail[k], its last m-tile
    if (k >= table[2 * E + 2]) return false;
    const int e = table[2 * E + 3 + k];
    g.e = e;
    g.nt = (lin - heads) - k * NT;
    g.m0 = expert_off[e] + (scan[e + 1] - scan[e]) * BM;
    g.mrows = expert_off[e + 1] - g.m0;
    return true;
  }
  int lo = 0, hi = E;  // scan[lo] * NT <= lin < scan[hi] * NT
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (scan[mid] * NT <= lin) lo = mid;
    else hi = mid;
  }
  const int me = scan[lo + 1] - scan[lo];  // >= 1: tile lin lies in this expert('s head)
  int mt;
  raster_tile(lin - scan[lo] * NT, me, NT, mt, g.nt);
  g.e = lo;
  g.m0 = expert_off[lo] + mt * BM;
  g.mrows = min(BM, expert_off[lo + 1] - g.m0);
  return true;
}

// The four LDS buffers of a GEMM workgroup.
#define MOE_GEMM_LDS(L)                                              \
  __shared__ __attribute__((aligned(1024))) char L##_0[LDS_BUF];     \
  __shared__ __attribute__((aligned(1024))) char L##_1[LDS_BUF];     \
  __shared__ __attribute__((aligned(1024))) char L##_2[LDS_BUF];     \
  __shared__ __attribute__((aligned(1024))) char L##_3[LDS_BUF];     \
  const LdsBufs L{{L##_0, L##_1, L##_2, L##_3}}

#define MOE_GEMM_LDS_HMX(L)                                          \
  __shared__ __attribute__((aligned(1024))) char L##_0[H_SLOT_MX];   \
  __shared__ __attribute__((aligned(1024))) char L##_1[H_SLOT_MX];   \
  __shared__ __attribute__((aligned(1024))) char L##_2[H_SLOT_MX]

#define MOE_GEMM_LDS_H(L)                                            \
  __shared__ __attribute__((aligned(1024))) char L##_0[H_SLOT];      \
  __shared__ __attribute__((aligned(1024))) char L##_1[H_SLOT];      \
  __shared__ __attribute__((aligned(1024))) char L##_2[H_SLOT]

}  // namespace moe

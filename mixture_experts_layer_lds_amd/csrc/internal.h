// Internal launcher interface between the C-ABI host layer (moe_api.cpp) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "common.h"

namespace moe {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct PlanPtrs {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* expert_off;
  int32_t* row_token;
  float* row_w;
  int32_t* tok_off;
  int32_t* tok_row;
  int32_t* meta;
};

// Problem description shared by the expert-GEMM launchers.
struct Shape {
  int64_t T, d, n;
  int E, K;
  int64_t R_max;
  bool bf16;  // element type of activations and weights (else fp32)
};

// ---- routing (route.hip) ----
size_t route_workspace_bytes(int64_t T, int E, bool rounded);
// part: null, or the SK - 1 partial products [SK-1][T][E] of a split router GEMM, which top-K adds
// to logits (in slice order) and writes back as the final logits before selecting.
hipError_t launch_route(float* logits, const float* part, int SK, int64_t T, int E, int K, int round_mode,
                        int tile_m, const uint32_t* round_rand, const PlanPtrs& p, void* ws, hipStream_t st);

// ---- grouped GEMM tile schedule (gemm_fwd.hip) ----
// The grouped GEMMs' tile table [tile_table_ints(E)]: the m-tiles per expert (scanned), and the
// same with the light tails (a last m-tile of 1..128 rows) listed apart so that a kernel can run
// them last (see find_group_tile); with order non-null also order[E]: experts by decreasing row
// count, ties to the lower id (the weight-gradient GEMMs' expert order, longest tiles first).
inline int tile_table_ints(int E) { return 3 * E + 3; }
hipError_t launch_tile_offsets(const int32_t* counts, int E, int32_t* mtile_off, int32_t* order, hipStream_t st);
int64_t max_mtiles(int64_t R_max, int E);

// ---- forward GEMMs (gemm_fwd.hip) ----
// logits[T,E] (fp32) = X[T,d] W_r[E,d]^T + bias.  With router_split(s) = SK > 1 (bf16 layers
// whose tiles would fill less than the chip) the reduction over d is cut into SK slices: slice 0
// (with the bias) goes to logits, slice q > 0 to part[q-1][T][E], and top-K adds them up.
int router_split(const Shape& s);
size_t router_part_bytes(const Shape& s);
hipError_t launch_router_gemm(const Shape& s, const void* X, const void* W_r, const float* bias,
                              float* logits, float* part, hipStream_t st);
// Act[R,n] = silu(G) * U with [G|U] = X[rows] [W_gate|W_up]^T; H[R,2n] optional
hipError_t launch_up_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                          const void* A_in, bool gathered, const void* W_gate, const void* W_up,
                          void* act, void* H, hipStream_t st);
// Y[R,d] = Act[R,n] W_down[e]^T
hipError_t launch_down_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                            const void* act, const void* W_down, void* Y, hipStream_t st);

// ---- FP8 expert FFN (fp8.hip) ----
// codes/scales of rows x K elements (rows_dev: optional device row bound, e.g. the plan's R)
hipError_t launch_quant_fp8(const void* src, bool is_bf16, int64_t rows, int64_t K, const int32_t* rows_dev,
                            uint8_t* codes, float* scales, hipStream_t st);
hipError_t launch_up_fp8(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, const uint8_t* Xq,
                         const float* sx, const uint8_t* Wgq, const float* sg, const uint8_t* Wuq,
                         const float* su, void* act, hipStream_t st);
hipError_t launch_down_fp8(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, const uint8_t* Aq,
                           const float* sa, const uint8_t* Wdq, const float* sd, void* Y, hipStream_t st);

// ---- block-scaled FP8 expert FFN (fp8.hip): E4M3 (fmt 0) or E5M2 (fmt 1) codes, one E8M0 scale
// byte per 32 elements along K, scales group-major [ceil(K / 128)][rows][4 bytes] ----
int64_t mx_scale_bytes(int64_t rows, int64_t K);
hipError_t launch_quant_mx(const void* src, bool is_bf16, int fmt, int64_t rows, int64_t K, uint8_t* codes,
                           uint8_t* scales, hipStream_t st);
// sxp = the token scales in routed-row order ([groups of d][R_max][4 B])
hipError_t launch_gather_mx_scales(const Shape& s, const PlanPtrs& p, const uint8_t* sx, uint8_t* sxp,
                                   hipStream_t st);
// act_q / sact ([groups of n][R_max][4 B]): the activation quantised in the gate/up epilogue;
// act (bf16) optional
hipError_t launch_up_mx(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, int fmt, const uint8_t* Xq,
                        const uint8_t* sxp, const uint8_t* Wgq, const uint8_t* sg, const uint8_t* Wuq,
                        const uint8_t* su, void* act, uint8_t* act_q, uint8_t* sact, hipStream_t st);
hipError_t launch_down_mx(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off, int fmt, const uint8_t* Aq,
                          const uint8_t* sa, const uint8_t* Wdq, const uint8_t* sd, void* Y, hipStream_t st);

// ---- permute / combine (combine.hip) ----
hipError_t launch_permute(const Shape& s, const PlanPtrs& p, const void* X, void* X_perm, hipStream_t st);
hipError_t launch_combine(const Shape& s, const PlanPtrs& p, const void* Y_perm, bool weighted,
                          void* out, hipStream_t st);

// ---- backward (backward.hip) ----
// dAct GEMM with the SwiGLU backward and dS partials in its epilogue:
//   dA' = dY[rows] W_down[e]   (N = n);  dS_part[nt][r] = sum over the tile's columns of dA' * A
//   dH[r] = [dG | dU];  wA[r] = w_r * A_r
hipError_t launch_dact_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                            const void* dY, const void* W_down, const void* H, void* dH, void* wA,
                            float* dS_part, hipStream_t st);
int dact_ntiles(int64_t n);
// dX_perm[R,d] = dG W_gate[e] + dU W_up[e]
hipError_t launch_dx_gemm(const Shape& s, const PlanPtrs& p, const int32_t* mtile_off,
                          const void* dH, const void* W_gate, const void* W_up, void* dX_perm,
                          hipStream_t st);
// dW_down[e] = (w dY[rows])^T A = dY[rows]^T wA, experts taken in `order`
hipError_t launch_dw_down_gemm(const Shape& s, const PlanPtrs& p, const int32_t* order, const void* dY,
                               const void* wA, void* dW_down, hipStream_t st);
// dW_gate[e] | dW_up[e] = dH^T X[rows], experts taken in `order`
hipError_t launch_dw_gu_gemm(const Shape& s, const PlanPtrs& p, const int32_t* order, const void* dH,
                             const void* X, void* dW_gate, void* dW_up, hipStream_t st);
// Router backward + dX gather-sum, one wave per token:
//   dS[r] = sum of partials; dL = w (dS - <w, dS>); dLogits row; dLop[t][e] (GEMM operand);
//   dX[t] = sum_r dX_perm[r] (+ sum_r dL_r W_r[e_r] if W_r)
hipError_t launch_router_bwd(const Shape& s, const PlanPtrs& p, const float* dS_part, int ntiles,
                             const void* dX_perm, const void* W_r, float* dS, float* dLogits,
                             void* dLop, int E_pad, void* dX, hipStream_t st);
// dW_r[E,d] = dL^T X (split over tokens, fp32 partials, fixed-order reduction)
size_t dwr_workspace_bytes(const Shape& s);
hipError_t launch_dwr_gemm(const Shape& s, const void* dLop, int E_pad, const void* X, void* dW_r,
                           void* ws, hipStream_t st);

// single-launch forward for small T (decode.hip)
size_t decode_workspace_bytes(int64_t T, int64_t d, int64_t n, int E, int K);
hipError_t launch_decode(const Shape& s, const void* X, const void* W_r, const float* bias,
                         const void* W_gate, const void* W_up, const void* W_down, float* logits,
                         int32_t* topk_idx, float* topk_w, void* out, void* ws, hipStream_t st);
// polls before a decode grid barrier gives up (later launches); returns the previous limit
long long decode_set_spin_limit(long long limit);
// synchronises st, then reads and clears the current device's decode status word (1 = a
// workgroup gave up at a grid barrier since the last read)
hipError_t decode_read_status(hipStream_t st, int* failed);

}  // namespace moe

/*
 * moe.h — C ABI of the MI355X (gfx950) Mixture-of-Experts layer library (libmoe_mi355x.so).
 *
 * One GPU runs the whole layer on its tokens: router logits, top-K, optional token rounding,
 * per-expert counts and offsets, the token permutation, grouped SwiGLU expert GEMMs with the row
 * gather fused into operand staging, the gate-weighted combine, and the backward pass.
 *
 * Where the operations come from (the pages this library implements):
 *  - cloud.baidu.com, "MoE架构的物理瓶颈与扩展限制解析", section "工作原理": the forward is
 *    gate network -> top-k -> dispatch -> local expert compute -> combine back to the tokens.
 *    With every expert on one GPU, dispatch and combine are a local row gather and a local sum.
 *  - apxml.com, "硬件加速的考量", section "自定义核与核融合": the five fused steps
 *    (gate scores, top-k, gather of the selected experts, expert matmuls, weighted combine).
 *  - hebangwen.github.io, "SonicMoE: 加速 MoE 模型的 IO 与 Tile 感知优化": gather fused into
 *    the GEMM's operand load ("Gather 与加载融合"; contiguous-packed or gathered inputs),
 *    SwiGLU fused into the GEMM, the router-score gradient computed without caching expert
 *    outputs, no separate scatter kernel (kernel-comparison table), recompute in the backward
 *    (optimization 1), and token rounding of per-expert counts to tile multiples
 *    (optimization 3).
 *
 * Conventions for every call:
 *  - Pointers are DEVICE pointers unless the comment says "host".  Tensors are dense row-major,
 *    with the shapes given below.  Every device pointer must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the legacy default stream).  All work is
 *    enqueued on it asynchronously; no call synchronises with the device, and data-dependent
 *    sizes (rows per expert, the total row count R) stay on the device.
 *  - The caller owns all memory: inputs, outputs, the routing plan and the workspace.  The
 *    library never allocates or frees device memory and keeps no state between calls, apart from
 *    a thread-local error message, when enabled the stage-timing records (moe_timing_*), and for
 *    moe_decode a per-device status word (static device memory, see moe_decode_status).
 *    Outputs are fully overwritten, never accumulated into.
 *  - Arguments are validated on the host before anything is enqueued.  An invalid call returns
 *    MOE_EINVAL / MOE_ENOTSUP / MOE_EWORKSPACE and enqueues nothing; a failed launch returns
 *    MOE_EHIP.  Faults inside kernels surface at the caller's next synchronisation, as in HIP.
 *    moe_last_error() returns a message describing the last failure on the calling thread.
 *  - Results are deterministic: the same inputs give bitwise-identical outputs (no floating-point
 *    atomics; every sum has a fixed order).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* a pointer is NULL/misaligned or a size is out of range */
  MOE_ENOTSUP = -2,    /* valid but unsupported shape or dtype (see moe_dims) */
  MOE_EWORKSPACE = -3, /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_EHIP = -4        /* the HIP runtime reported an error when launching */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Token rounding (SonicMoE page, optimization 3).  Each expert's token count c is moved to a
 * multiple of tile_m: NEAREST drops r = c mod tile_m tokens when r < tile_m/2 and otherwise adds
 * tile_m - r (half a tile rounds up); UP always adds; DOWN always drops; STOCHASTIC adds with
 * probability r / tile_m using the caller's random words (moe_dims.round_rand), which keeps the
 * expected count; an addition that would need more than T tokens drops instead.  An expert drops its lowest-ranked members and adds its
 * highest-ranked non-members, ranking tokens by (logit descending, token id ascending). */
typedef enum {
  MOE_ROUND_NONE = 0,
  MOE_ROUND_NEAREST = 1,
  MOE_ROUND_UP = 2,
  MOE_ROUND_DOWN = 3,
  MOE_ROUND_STOCHASTIC = 4
} moe_round;

/* Layer shape (host struct).
 *  T tokens (1 .. 2^24), d model width, n expert FFN width (d and n multiples of 64,
 *  64 .. 65536), E experts (1 .. 1024), K experts per token (1 .. min(E, 16)).
 *  dtype: type of X, W_r, W_gate, W_up, W_down, dY, out, dX, dW_*, H and Y_perm.  Logits, gate
 *  weights, dS and dLogits are always fp32; accumulation is always fp32.
 *  round_mode / tile_m: token rounding (tile_m 1 .. 1024; ignored for MOE_ROUND_NONE).
 *  flags: reserved, must be 0.
 *  round_rand: device array [E] of uniform 32-bit random words, read only by
 *   MOE_ROUND_STOCHASTIC (must then be non-NULL): expert e with r = count mod tile_m != 0 rounds
 *   up iff round_rand[e] * tile_m < r * 2^32, i.e. with probability r / tile_m, so its expected
 *   count is unchanged (SonicMoE optimization 3 keeps the expected total); otherwise it drops r
 *   tokens as DOWN does.  The caller draws fresh words per call; the library owns no generator. */
typedef struct moe_dims {
  int64_t T;
  int64_t d;
  int64_t n;
  int32_t E;
  int32_t K;
  int32_t dtype;
  int32_t round_mode;
  int32_t tile_m;
  int32_t flags;
  const uint32_t* round_rand;
} moe_dims;

/* The routing plan: device arrays the caller allocates with the sizes given here, written by
 * moe_route and read by the other calls.  R is the number of (token, expert) rows after token
 * rounding; R_max = moe_max_rows(dims) bounds it.  Row r of the permuted ("expert-major") layout
 * belongs to expert e when expert_off[e] <= r < expert_off[e+1]; an expert's rows are its tokens
 * in ascending token id.
 *   topk_idx   int32 [T*K]   plain top-K expert ids per token, best first (ties: lower id)
 *   topk_w     fp32  [T*K]   softmax of the token's K selected logits (plain top-K weights)
 *   counts     int32 [E]     rows per expert after token rounding
 *   expert_off int32 [E+1]   exclusive prefix sum of counts; expert_off[E] = R
 *   row_token  int32 [R_max] token of row r (entries r >= R are unspecified)
 *   row_w      fp32  [R_max] gate weight of row r: softmax over the token's final experts
 *   tok_off    int32 [T+1]   token t owns tok_row[tok_off[t] .. tok_off[t+1])
 *   tok_row    int32 [R_max] rows of each token, in ascending expert id
 *   meta       int32 [16]    meta[0] = R; the other entries are reserved */
typedef struct moe_plan {
  int32_t* topk_idx;
  float* topk_w;
  int32_t* counts;
  int32_t* expert_off;
  int32_t* row_token;
  float* row_w;
  int32_t* tok_off;
  int32_t* tok_row;
  int32_t* meta;
} moe_plan;

/* Operation codes for moe_workspace_bytes(). */
enum {
  MOE_OP_ROUTE = 0,
  MOE_OP_PERMUTE = 1,
  MOE_OP_FFN = 2,
  MOE_OP_COMBINE = 3,
  MOE_OP_FORWARD = 4,
  MOE_OP_BACKWARD = 5,
  MOE_OP_DECODE = 6,
  MOE_OP_FFN_FP8 = 7,
  MOE_OP_FFN_MX = 8
};

/* Host: upper bound on R for these dims (T*K without rounding; rounding can add at most
 * tile_m - 1 rows per expert, and never more than T*E rows in total).  0 if dims are invalid. */
int64_t moe_max_rows(const moe_dims* dims);

/* Host: workspace bytes the call `op` needs for these dims (0 if none; 0 for invalid dims, with
 * moe_last_error() set).  A workspace may be reused by calls that are ordered on one stream. */
size_t moe_workspace_bytes(const moe_dims* dims, int op);

/* moe_route — gate network, top-K, token rounding, counts, offsets and the permutation indices.
 * cloud.baidu.com "工作原理" steps 1 (gate_network, top_k); apxml.com fused steps 1-2; SonicMoE
 * optimization 3 (token rounding).
 *  X      [T,d] dtype, W_r [E,d] dtype, bias [E] fp32 or NULL: if X != NULL, the library computes
 *         logits = X W_r^T + bias (fp32 accumulation) and writes them to `logits`; a bf16 layer
 *         with fewer than 256 tiles of 256 tokens x 128 experts sums d in 2 or 4 slices, added
 *         in slice order (a fixed order: the result does not depend on the schedule).
 *         If X == NULL, `logits` is an INPUT: caller-computed fp32 logits (bias already added).
 *  logits [T,E] fp32.  NaN ranks below every number (so a token still gets K distinct experts).
 *  plan   all arrays written (see moe_plan).
 * Selection compares fp32 logits exactly: the K largest per token (ties to the lower expert id);
 * the gate weights are the softmax over the token's final expert set.  A token that token
 * rounding leaves with no expert has no rows. */
moe_status moe_route(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                     float* logits, const moe_plan* plan, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_route_noalloc — moe_route with its workspace in a static device buffer of the library
 * instead of a caller workspace: for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  Arguments, outputs and
 * results are those of moe_route; the call itself allocates nothing.
 *  Limit: moe_workspace_bytes(dims, MOE_OP_ROUTE) must not exceed moe_route_noalloc_max_bytes()
 *  (64 MiB; e.g. T = 32768 tokens with E = 384 experts and token rounding need 51 MiB), else
 *  MOE_EWORKSPACE and nothing is enqueued.
 *  The buffer: one copy per device, held until the process ends; its address is looked up on
 *  the first call on each device.  No part of it needs to start at zero.  Every call on a device
 *  shares that device's copy, so calls that may overlap on one device (other streams, other host
 *  threads) race and corrupt each other's plans: order them on one stream. */
moe_status moe_route_noalloc(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                             float* logits, const moe_plan* plan, void* stream);
/* Host: size in bytes of moe_route_noalloc's static buffer. */
size_t moe_route_noalloc_max_bytes(void);

/* moe_permute — materialise the expert-major copy of the tokens ("contiguous packed" input):
 * X_perm[r] = X[row_token[r]] for r < R.  X [T,d] dtype, X_perm [R_max,d] dtype (rows >= R are
 * left untouched).  Bit-exact copies.  Needs a plan from moe_route. */
moe_status moe_permute(const moe_dims* dims, const moe_plan* plan, const void* X, void* X_perm,
                       void* stream);

/* moe_grouped_ffn — every expert's SwiGLU FFN on its rows, as grouped GEMMs.
 *  A_in     gathered != 0: X [T,d]; row r reads X[row_token[r]] straight into the GEMM's operand
 *           staging (no permuted copy).  gathered == 0: X_perm [R_max,d] from moe_permute.
 *  W_gate, W_up [E,n,d] dtype;  W_down [E,d,n] dtype.
 *  H_cache  [R_max,2n] dtype or NULL: if given, row r receives [G_r | U_r] with
 *           G = x W_gate[e]^T and U = x W_up[e]^T (the pre-activations the backward reuses).
 *  Y_perm   [R_max,d] dtype: Y_r = (silu(G_r) * U_r) W_down[e]^T.
 * silu(g) = g / (1 + exp(-g)).  fp32 accumulation; the SwiGLU output is rounded to dtype between
 * the two GEMMs. */
moe_status moe_grouped_ffn(const moe_dims* dims, const moe_plan* plan, const void* A_in,
                           int gathered, const void* W_gate, const void* W_up,
                           const void* W_down, void* H_cache, void* Y_perm, void* ws,
                           size_t ws_bytes, void* stream);

/* moe_combine — scatter-free combine: out[t] = sum over the token's rows r (ascending expert)
 * of w_r * Y_perm[r], with w_r = row_w[r] if weighted != 0, else 1.  fp32 accumulation, one
 * rounding to dtype.  A token with no rows gets zeros.  Y_perm [R_max,d], out [T,d] dtype. */
moe_status moe_combine(const moe_dims* dims, const moe_plan* plan, const void* Y_perm,
                       int weighted, void* out, void* stream);

/* moe_forward — the whole layer: moe_route (logits from X, W_r, bias), the grouped FFN on
 * gathered rows, and the weighted combine.
 *  logits [T,E] fp32 output; plan output; H_cache [R_max,2n] or NULL (see moe_grouped_ffn);
 *  out [T,d] dtype. */
moe_status moe_forward(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                       const void* W_gate, const void* W_up, const void* W_down, float* logits,
                       const moe_plan* plan, void* H_cache, void* out, void* ws,
                       size_t ws_bytes, void* stream);

/* moe_backward — gradients of the layer for the routing in `plan` (selection and token rounding
 * held fixed; the bias is a constant).  SonicMoE optimization 1 and "反向传播优化".
 *  dY [T,d] dtype: gradient of the loss with respect to out.
 *  X, W_gate, W_up, W_down: the forward's inputs.  plan: the forward's plan.
 *  H_cache [R_max,2n] from the forward, or NULL: then [G|U] is recomputed from X first.
 *  The SwiGLU output A = silu(G) * U is recomputed from H; expert outputs Y are never needed:
 *  dS_r = <dY[t_r] W_down[e], A_r> equals <dY[t_r], Y_r>.
 *  Outputs (all overwritten):
 *   dX [T,d] dtype           expert-path gradient plus, if W_r != NULL, dLogits W_r
 *   dW_gate, dW_up [E,n,d], dW_down [E,d,n] dtype  (zero for experts without rows)
 *   dS [R_max] fp32          dLoss/dw_r per row (rows >= R unspecified)
 *   dLogits [T,E] fp32       w_j (dS_j - sum_k w_k dS_k) on the token's experts, 0 elsewhere
 *   dW_r [E,d] dtype or NULL (requires W_r): dLogits^T X */
moe_status moe_backward(const moe_dims* dims, const void* dY, const void* X, const void* W_r,
                        const void* W_gate, const void* W_up, const void* W_down,
                        const moe_plan* plan, const void* H_cache, void* dX, void* dW_gate,
                        void* dW_up, void* dW_down, float* dS, float* dLogits, void* dW_r,
                        void* ws, size_t ws_bytes, void* stream);

/* moe_decode — the whole forward layer in one kernel launch, for small token counts (decode /
 * inference): router logits, top-K with softmax, the selected experts' SwiGLU FFNs and the
 * weighted combine.  apxml.com "自定义核与核融合" (the five steps fused into one kernel) and
 * "条件参数加载" (only the selected experts' weights are read, each once per 48 routed tokens).
 * Plain top-K only (round_mode must be MOE_ROUND_NONE, else MOE_ENOTSUP); T <= 1024.  The
 * grid is one workgroup per CU, phases separated by grid-wide barriers, so the whole grid must
 * be resident at once: it is on a device that runs nothing else; if other work (other streams)
 * holds CUs for longer than the barrier bound below, the call fails as described there instead
 * of hanging.  The barriers count arrivals in the call's workspace, which a small kernel clears right
 * before the launch, so calls share no device state: calls that may overlap (other streams) need
 * only their own workspaces.  A barrier wait is bounded (about a second of polling; see
 * moe_decode_set_spin_limit); a workgroup that reaches the bound leaves the kernel and sets the
 * device's decode status word, the other workgroups give up at the next barrier, and the call's
 * outputs are then invalid: moe_decode_status() reports it.  Results
 * equal moe_forward's with plain top-K up to the order of the fp32 accumulations (the SwiGLU
 * activation is rounded to dtype between the projections, as in moe_forward); routing is the
 * same function of the logits, ties to the lower expert id.  It pays off while few experts
 * see each a few tokens and their weights are large (on MI355X it beats moe_forward at T = 1
 * and T = 8 on the layer shapes with large experts, and at T = 1 on the fine-grained shape:
 * d = 1536, n = 256); once most experts are routed with several tokens each (T = 64 on the
 * large-expert shapes), or at T >= 8 on the fine-grained shape, moe_forward is as fast or
 * faster.
 *  X [T,d], W_r [E,d], bias [E] fp32 or NULL, W_gate/W_up [E,n,d], W_down [E,d,n] dtype.
 *  Outputs (overwritten): logits [T,E] fp32, topk_idx [T,K] int32, topk_w [T,K] fp32 (as in the
 *  plan of moe_route), out [T,d] dtype.
 *  ws: moe_workspace_bytes(dims, MOE_OP_DECODE) bytes (barrier counter, per-expert token lists,
 *  the activation and the fp32 expert outputs of the T*K (token, expert) pairs); contents on
 *  entry unused. */
moe_status moe_decode(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                      const void* W_gate, const void* W_up, const void* W_down, float* logits,
                      int32_t* topk_idx, float* topk_w, void* out, void* ws, size_t ws_bytes,
                      void* stream);

/* moe_decode_status — host: waits for `stream` (hipStreamSynchronize), then reads and clears the
 * current device's decode status word.  Returns MOE_EHIP (with a message) if a moe_decode kernel
 * on this device gave up waiting at a grid barrier since the last call, so that its outputs are
 * invalid; MOE_OK otherwise; MOE_EHIP also if the runtime fails. */
moe_status moe_decode_status(void* stream);

/* moe_decode_set_spin_limit — host: polls of the counter before a moe_decode grid barrier gives
 * up, for launches made after this call (default 2^20, about a second; 0 gives up at the first
 * barrier without waiting, which exercises the failure report).  Returns the previous limit, or
 * -1 (MOE_EINVAL in moe_last_error) for a negative limit.  Not thread-safe. */
long long moe_decode_set_spin_limit(long long limit);

/* moe_quantize_fp8 — per-row FP8 quantisation (apxml.com "硬件加速的考量", section "利用稀疏性和
 * 量化": FP8 weights and activations).  Format: OCP FP8 E4M3 codes (bias 7, largest finite 448,
 * no infinities), one fp32 scale per row: the smallest power of two s with max|row| / s <= 448
 * (s = 1 for a row of zeros); code = the nearest E4M3 value to x / s, ties to even.  Value of an
 * element = decode(code) * s.
 *  src [rows, K] dtype (MOE_BF16 or MOE_F32), rows >= 0, K a positive multiple of 8; finite
 *  values (results for NaN / infinity are unspecified).  codes [rows, K] uint8 and scales [rows]
 *  fp32, overwritten.  Weights are quantised once with this call (W_gate / W_up as [E*n, d],
 *  W_down as [E*d, n]); moe_grouped_ffn_fp8 quantises its activation itself. */
moe_status moe_quantize_fp8(int64_t rows, int64_t K, int dtype, const void* src, uint8_t* codes,
                            float* scales, void* stream);

/* moe_grouped_ffn_fp8 — the experts' SwiGLU FFN with FP8 (E4M3, per-row scales, see
 * moe_quantize_fp8) operands on gathered token rows: MFMA on the codes with fp32 accumulation,
 * scales applied to the sums.  dims.dtype must be MOE_BF16 (the activation and Y_perm are bf16).
 *  Xq [T,d] uint8 + sx [T] fp32: the tokens, quantised per row;
 *  Wg_q, Wu_q [E,n,d] uint8 + sg, su [E,n] fp32;  Wd_q [E,d,n] uint8 + sd [E,d] fp32.
 *  Outputs (rows r < R of the plan; rows past R untouched):
 *    act   [R_max,n] bf16: silu(G_r) U_r with G = s_x s_g (xq wg_q^T), U likewise;
 *    act_q [R_max,n] uint8 + sact [R_max] fp32: act quantised per row;
 *    Y_perm [R_max,d] bf16: Y_r = s_a s_d (act_q wd_q^T).
 *  ws: moe_workspace_bytes(dims, MOE_OP_FFN_FP8) bytes. */
moe_status moe_grouped_ffn_fp8(const moe_dims* dims, const moe_plan* plan, const uint8_t* Xq,
                               const float* sx, const uint8_t* Wg_q, const float* sg,
                               const uint8_t* Wu_q, const float* su, const uint8_t* Wd_q,
                               const float* sd, void* act, uint8_t* act_q, float* sact,
                               void* Y_perm, void* ws, size_t ws_bytes, void* stream);

/* Block-scaled FP8 (apxml.com "硬件加速的考量", section "利用稀疏性和量化": FP8 weights and
 * activations).  Element format OCP FP8 E4M3 (bias 7, largest finite 448, no infinities) or E5M2
 * (bias 15, largest finite 57344); each row of an operand is cut along its reduction dimension K
 * into blocks of 32 consecutive elements, and each block has one scale s = 2^(byte - 127) (an
 * E8M0 byte): the smallest power of two with max|block| / s <= the format's largest finite
 * value, s = 1 for an all-zero block, kept within 2^-127 .. 2^127.  Element codes are the nearest
 * code to x / s, ties to even.  The GEMMs apply the block scales inside the MFMA
 * (v_mfma_scale_f32_32x32x64_f8f6f4), so every product is exact before the fp32 accumulation.
 * Scales are stored group-major: a group is the four blocks of 128 consecutive elements of a row,
 * and groups are planes of one 4-byte word per row, so the scale byte of block b of row r in a
 * matrix of `rows` rows is at byte (b / 4) * rows * 4 + r * 4 + b % 4 (the GEMMs load the words of
 * 64 consecutive rows as one 256-byte access).  Bytes of blocks past K / 32 are unspecified. */
typedef enum { MOE_FP8_E4M3 = 0, MOE_FP8_E5M2 = 1 } moe_fp8_format;

/* Host: bytes of block scales for a rows x K matrix: ceil(K / 128) * rows * 4 (0 if invalid). */
int64_t moe_mx_scale_bytes(int64_t rows, int64_t K);

/* moe_quantize_mx — block-scaled quantisation of a rows x K matrix (K a multiple of 64, at most
 * 65536).  src [rows, K] dtype (MOE_BF16 or MOE_F32), finite values; fmt a moe_fp8_format.
 * codes [rows, K] uint8 and scales (moe_mx_scale_bytes(rows, K) bytes, group-major) overwritten.  Weights
 * are quantised once with this call (W_gate / W_up as [E*n, d], W_down as [E*d, n]), tokens
 * every step; moe_grouped_ffn_mx quantises its activation itself. */
moe_status moe_quantize_mx(int64_t rows, int64_t K, int dtype, int fmt, const void* src, uint8_t* codes,
                           uint8_t* scales, void* stream);

/* moe_grouped_ffn_mx — the experts' SwiGLU FFN on block-scaled FP8 operands (format fmt for all
 * of them) and gathered token rows.  dims.dtype must be MOE_BF16; T * d must be below 2^32.
 *  Xq [T,d] + sx (scales of T rows of d);  Wg_q, Wu_q [E,n,d] + sg, su (scales of E*n rows of d);
 *  Wd_q [E,d,n] + sd (scales of E*d rows of n); scales group-major as above.
 *  The gate/up GEMM forms act = silu(G) U per row r (G, U accumulated in fp32 from exact block
 *  products), rounds it to bf16 and quantises it in its epilogue, 32 columns to a block:
 *    act   [R_max,n] bf16 or NULL (written when given: the activation before quantisation);
 *    act_q [R_max,n] uint8 + sact (scales of R_max rows of n): its codes and scales;
 *  then Y_perm [R_max,d] bf16: Y_r = act_q_r Wd_q[e]^T with both operands' block scales.
 *  Rows r < R of the plan are written; rows past R are untouched.
 *  ws: moe_workspace_bytes(dims, MOE_OP_FFN_MX) bytes. */
moe_status moe_grouped_ffn_mx(const moe_dims* dims, const moe_plan* plan, int fmt, const uint8_t* Xq,
                              const uint8_t* sx, const uint8_t* Wg_q, const uint8_t* sg, const uint8_t* Wu_q,
                              const uint8_t* su, const uint8_t* Wd_q, const uint8_t* sd, void* act,
                              uint8_t* act_q, uint8_t* sact, void* Y_perm, void* ws, size_t ws_bytes,
                              void* stream);

/* Stages of the layer, for the timing facility below.  Each stage is one kernel, except ROUTE
 * (top-K, counts, token rounding, offsets, placement) and DWR_GEMM (GEMM + slice reduction). */
typedef enum {
  MOE_STAGE_ROUTER_GEMM = 0, /* logits = X W_r^T + bias */
  MOE_STAGE_ROUTE = 1,       /* top-K ... placement */
  MOE_STAGE_TILES = 2,       /* grouped-GEMM tile offsets */
  MOE_STAGE_UP_GEMM = 3,     /* gate/up GEMM + SwiGLU (also the backward's recompute) */
  MOE_STAGE_DOWN_GEMM = 4,   /* down GEMM */
  MOE_STAGE_PERMUTE = 5,     /* materialised permute */
  MOE_STAGE_COMBINE = 6,     /* weighted combine */
  MOE_STAGE_DACT_GEMM = 7,   /* backward dAct GEMM + SwiGLU backward + dS partials */
  MOE_STAGE_DW_DOWN_GEMM = 8,
  MOE_STAGE_DW_GU_GEMM = 9,
  MOE_STAGE_DX_GEMM = 10,
  MOE_STAGE_ROUTER_BWD = 11, /* dS, dLogits and the dX gather-sum */
  MOE_STAGE_DWR_GEMM = 12,
  MOE_STAGE_DECODE = 13,     /* the single-launch forward of moe_decode */
  MOE_STAGE_FP8_QUANT = 14,  /* FP8 row quantisation (moe_quantize_fp8 and the activation's) */
  MOE_STAGE_FP8_UP = 15,     /* FP8 gate/up GEMM + SwiGLU */
  MOE_STAGE_FP8_DOWN = 16,   /* FP8 down GEMM */
  MOE_STAGE_COUNT = 17
} moe_stage;

/* Host: stage timing for measurement tools (not thread-safe; for a single host thread).
 * moe_timing_enable(1) makes every later call record a hipEvent pair around each stage it
 * enqueues, on the call's stream, up to 4096 stage launches; moe_timing_enable(0) stops
 * recording and releases the events (it synchronises with them first).  Returns MOE_OK or
 * MOE_EHIP.  moe_timing_read(stage, ms, max) waits for the recorded events and writes the
 * durations of that stage's launches (in launch order, milliseconds) to ms[0..]; it returns how
 * many it wrote (at most max), or a negative moe_status.  Recording starts empty at every
 * moe_timing_enable(1). */
int moe_timing_enable(int on);
int moe_timing_read(int stage, float* ms, int max);

/* Host: static text for a status code. */
const char* moe_status_string(int status);
/* Host: message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);
/* Host: library version string. */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */

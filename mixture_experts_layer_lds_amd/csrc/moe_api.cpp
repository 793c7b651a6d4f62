// C ABI of the MoE layer library: argument validation, workspace layout and the launch sequence
// of each call.  Every call validates everything on the host before it enqueues anything, then
// enqueues its kernels on the caller's stream without synchronising.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/moe.h"
#include "internal.h"

using namespace moe;

namespace {

thread_local std::string g_err;

moe_status fail(moe_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

moe_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return MOE_OK;
  return fail(MOE_EHIP, "%s: HIP error %d (%s)", where, (int)e, hipGetErrorString(e));
}

#define MOE_TRY(expr)                      \
  do {                                     \
    moe_status _s = (expr);                \
    if (_s != MOE_OK) return _s;           \
  } while (0)
#define MOE_HIP(expr, where) MOE_TRY(hip_status((expr), (where)))

// ---- stage timing (moe_timing_enable / moe_timing_read) ----
constexpr int kTimingSlots = 4096;
struct Timing {
  bool on = false;
  int used = 0;
  int stage[kTimingSlots];
  hipEvent_t ev0[kTimingSlots];
  hipEvent_t ev1[kTimingSlots];
  bool created = false;
};
Timing g_timing;

// Record the start of a stage: the slot, or -1 when timing is off or the slots are used up.
hipError_t stage_begin(int stage, hipStream_t st, int* slot) {
  *slot = -1;
  if (!g_timing.on || g_timing.used >= kTimingSlots) return hipSuccess;
  const int i = g_timing.used;
  const hipError_t e = hipEventRecord(g_timing.ev0[i], st);
  if (e != hipSuccess) return e;
  g_timing.stage[i] = stage;
  g_timing.used = i + 1;
  *slot = i;
  return hipSuccess;
}
hipError_t stage_end(int slot, hipStream_t st) {
  return slot >= 0 ? hipEventRecord(g_timing.ev1[slot], st) : hipSuccess;
}

// Run one stage's launcher between timing events; a failed launch or event record is MOE_EHIP.
#define MOE_STAGE(stage, st, expr, where)                      \
  do {                                                         \
    int _slot;                                                 \
    MOE_HIP(stage_begin((stage), (st), &_slot), "timing event"); \
    const hipError_t _e = (expr);                              \
    MOE_HIP(_e, where);                                        \
    MOE_HIP(stage_end(_slot, (st)), "timing event");           \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status need_ptr(const void* p, const char* name) {
  if (!p) return fail(MOE_EINVAL, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_EINVAL, "%s is not 16-byte aligned", name);
  return MOE_OK;
}
moe_status opt_ptr(const void* p, const char* name) {
  if (p && !aligned16(p)) return fail(MOE_EINVAL, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

moe_status check_dims(const moe_dims* dm) {
  if (!dm) return fail(MOE_EINVAL, "dims is NULL");
  if (dm->T < 1 || dm->T > (1 << 24)) return fail(MOE_EINVAL, "T=%lld out of range [1, 2^24]", (long long)dm->T);
  if (dm->E < 1 || dm->E > 1024) return fail(MOE_EINVAL, "E=%d out of range [1, 1024]", dm->E);
  if (dm->K < 1 || dm->K > dm->E) return fail(MOE_EINVAL, "K=%d out of range [1, E=%d]", dm->K, dm->E);
  if (dm->K > 16) return fail(MOE_ENOTSUP, "K=%d > 16 is not supported", dm->K);
  if (dm->d < 64 || dm->d > 65536 || dm->n < 64 || dm->n > 65536)
    return fail(MOE_EINVAL, "d=%lld / n=%lld out of range [64, 65536]", (long long)dm->d, (long long)dm->n);
  if (dm->d % 64 || dm->n % 64)
    return fail(MOE_ENOTSUP, "d=%lld and n=%lld must be multiples of 64", (long long)dm->d, (long long)dm->n);
  if (dm->dtype != MOE_F32 && dm->dtype != MOE_BF16) return fail(MOE_ENOTSUP, "dtype %d not supported", dm->dtype);
  if (dm->round_mode < MOE_ROUND_NONE || dm->round_mode > MOE_ROUND_STOCHASTIC)
    return fail(MOE_EINVAL, "round_mode %d invalid", dm->round_mode);
  if (dm->round_mode == MOE_ROUND_STOCHASTIC && !dm->round_rand)
    return fail(MOE_EINVAL, "MOE_ROUND_STOCHASTIC needs round_rand");
  if (dm->round_mode != MOE_ROUND_NONE && (dm->tile_m < 1 || dm->tile_m > 1024))
    return fail(MOE_EINVAL, "tile_m=%d out of range [1, 1024]", dm->tile_m);
  if (dm->flags != 0) return fail(MOE_EINVAL, "flags must be 0");
  return MOE_OK;
}

int64_t max_rows(const moe_dims* dm) {
  const int64_t base = dm->T * dm->K;
  if (dm->round_mode == MOE_ROUND_NONE || dm->round_mode == MOE_ROUND_DOWN) return base;
  const int64_t up = base + (int64_t)dm->E * (dm->tile_m - 1);
  const int64_t cap = dm->T * dm->E;
  return up < cap ? up : cap;
}

Shape shape_of(const moe_dims* dm) {
  Shape s;
  s.T = dm->T;
  s.d = dm->d;
  s.n = dm->n;
  s.E = dm->E;
  s.K = dm->K;
  s.R_max = max_rows(dm);
  s.bf16 = dm->dtype == MOE_BF16;
  return s;
}

size_t esize(const moe_dims* dm) { return dm->dtype == MOE_BF16 ? 2 : 4; }
int e_pad(int E) { return (E + 7) / 8 * 8; }

// Bump allocator over the workspace; with base == nullptr it only measures.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* b) : base(static_cast<char*>(b)) {}
  void* take(size_t bytes) {
    void* p = base ? base + off : nullptr;
    off = align_up(off + bytes, 256);
    return p;
  }
};

struct FfnWs {
  int32_t* mtile_off;
  void* act;
};
FfnWs carve_ffn(Carve& c, const moe_dims* dm) {
  FfnWs w;
  w.mtile_off = static_cast<int32_t*>(c.take((size_t)tile_table_ints(dm->E) * 4));
  w.act = c.take((size_t)max_rows(dm) * dm->n * esize(dm));
  return w;
}

struct BwdWs {
  int32_t* mtile_off;
  int32_t* order;
  void* H;
  void* dH;
  void* wA;
  float* dS_part;
  void* dX_perm;
  void* dLop;
  void* dwr;
};
BwdWs carve_bwd(Carve& c, const moe_dims* dm) {
  const Shape s = shape_of(dm);
  const size_t es = esize(dm);
  BwdWs w;
  w.mtile_off = static_cast<int32_t*>(c.take((size_t)tile_table_ints(dm->E) * 4));
  w.order = static_cast<int32_t*>(c.take((size_t)dm->E * 4));
  w.H = c.take((size_t)s.R_max * 2 * dm->n * es);
  w.dH = c.take((size_t)s.R_max * 2 * dm->n * es);
  w.wA = c.take((size_t)s.R_max * dm->n * es);
  w.dS_part = static_cast<float*>(c.take((size_t)dact_ntiles(dm->n) * s.R_max * 4));
  w.dX_perm = c.take((size_t)s.R_max * dm->d * es);
  w.dLop = c.take((size_t)dm->T * e_pad(dm->E) * es);
  w.dwr = c.take(dwr_workspace_bytes(s));
  return w;
}

size_t ws_bytes_for(const moe_dims* dm, int op) {
  Carve c(nullptr);
  switch (op) {
    case MOE_OP_ROUTE:  // (+ the partial products of a split router GEMM)
      return route_workspace_bytes(dm->T, dm->E, dm->round_mode != 0) + router_part_bytes(shape_of(dm));
    case MOE_OP_PERMUTE: return 0;
    case MOE_OP_COMBINE: return 0;
    case MOE_OP_FFN: carve_ffn(c, dm); return c.off;
    case MOE_OP_FORWARD: {
      carve_ffn(c, dm);
      c.take((size_t)max_rows(dm) * dm->d * esize(dm));  // Y_perm
      const size_t r = route_workspace_bytes(dm->T, dm->E, dm->round_mode != 0) + router_part_bytes(shape_of(dm));
      return c.off > r ? c.off : r;
    }
    case MOE_OP_BACKWARD: carve_bwd(c, dm); return c.off;
    case MOE_OP_DECODE: return decode_workspace_bytes(dm->T, dm->d, dm->n, dm->E, dm->K);
    case MOE_OP_FFN_FP8: c.take((size_t)tile_table_ints(dm->E) * 4); return c.off;
    case MOE_OP_FFN_MX:  // tile table, the token scales in routed-row order
      c.take((size_t)tile_table_ints(dm->E) * 4);
      c.take((size_t)mx_scale_bytes(max_rows(dm), dm->d));
      return c.off;
    default: return 0;
  }
}

moe_status check_plan(const moe_plan* p) {
  if (!p) return fail(MOE_EINVAL, "plan is NULL");
  MOE_TRY(need_ptr(p->topk_idx, "plan.topk_idx"));
  MOE_TRY(need_ptr(p->topk_w, "plan.topk_w"));
  MOE_TRY(need_ptr(p->counts, "plan.counts"));
  MOE_TRY(need_ptr(p->expert_off, "plan.expert_off"));
  MOE_TRY(need_ptr(p->row_token, "plan.row_token"));
  MOE_TRY(need_ptr(p->row_w, "plan.row_w"));
  MOE_TRY(need_ptr(p->tok_off, "plan.tok_off"));
  MOE_TRY(need_ptr(p->tok_row, "plan.tok_row"));
  MOE_TRY(need_ptr(p->meta, "plan.meta"));
  return MOE_OK;
}

PlanPtrs plan_ptrs(const moe_plan* p) {
  PlanPtrs q;
  q.topk_idx = p->topk_idx;
  q.topk_w = p->topk_w;
  q.counts = p->counts;
  q.expert_off = p->expert_off;
  q.row_token = p->row_token;
  q.row_w = p->row_w;
  q.tok_off = p->tok_off;
  q.tok_row = p->tok_row;
  q.meta = p->meta;
  return q;
}

moe_status check_ws(const moe_dims* dm, int op, void* ws, size_t ws_bytes) {
  const size_t need = ws_bytes_for(dm, op);
  if (need == 0) return MOE_OK;
  if (ws_bytes < need) return fail(MOE_EWORKSPACE, "workspace of %zu bytes < %zu needed", ws_bytes, need);
  return need_ptr(ws, "ws");
}

// The routing stage shared by moe_route and moe_forward (arguments already validated).
// With X the router GEMM runs first; when it splits its reduction (router_split), the partial
// products go to the end of the routing workspace and top-K adds them into logits.
moe_status do_route(const moe_dims* dm, const void* X, const void* W_r, const float* bias,
                    float* logits, const moe_plan* plan, void* ws, hipStream_t st) {
  const Shape s = shape_of(dm);
  const int SK = X ? router_split(s) : 1;
  float* part = SK > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                  route_workspace_bytes(dm->T, dm->E, dm->round_mode != 0))
                       : nullptr;
  if (X) MOE_STAGE(MOE_STAGE_ROUTER_GEMM, st, launch_router_gemm(s, X, W_r, bias, logits, part, st), "router GEMM");
  MOE_STAGE(MOE_STAGE_ROUTE, st,
            launch_route(logits, part, SK, dm->T, dm->E, dm->K, dm->round_mode, dm->tile_m, dm->round_rand,
                         plan_ptrs(plan), ws, st),
            "routing");
  return MOE_OK;
}

moe_status do_ffn(const moe_dims* dm, const moe_plan* plan, const void* A_in, bool gathered,
                  const void* Wg, const void* Wu, const void* Wd, void* H, void* Y, const FfnWs& w,
                  hipStream_t st) {
  const Shape s = shape_of(dm);
  const PlanPtrs p = plan_ptrs(plan);
  MOE_STAGE(MOE_STAGE_TILES, st, launch_tile_offsets(p.counts, dm->E, w.mtile_off, nullptr, st), "tile offsets");
  MOE_STAGE(MOE_STAGE_UP_GEMM, st, launch_up_gemm(s, p, w.mtile_off, A_in, gathered, Wg, Wu, w.act, H, st),
            "gate/up GEMM");
  MOE_STAGE(MOE_STAGE_DOWN_GEMM, st, launch_down_gemm(s, p, w.mtile_off, w.act, Wd, Y, st), "down GEMM");
  return MOE_OK;
}

// ---- allocation-free routing (moe_route_noalloc) ----
// The routing workspace of moe_route_noalloc: one copy per device, held until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory; kernels get the device
// address from hipGetSymbolAddress, resolved once per device.
constexpr size_t kRouteScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kRouteScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

moe_status route_scratch(void** out) {
  int dev = 0;
  MOE_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_EHIP, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

int64_t moe_max_rows(const moe_dims* dims) {
  if (check_dims(dims) != MOE_OK) return 0;
  return max_rows(dims);
}

size_t moe_workspace_bytes(const moe_dims* dims, int op) {
  if (check_dims(dims) != MOE_OK) return 0;
  if (op < MOE_OP_ROUTE || op > MOE_OP_FFN_MX) {
    fail(MOE_EINVAL, "unknown op %d", op);
    return 0;
  }
  return ws_bytes_for(dims, op);
}

moe_status moe_route(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                     float* logits, const moe_plan* plan, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(logits, "logits"));
  if (X) {
    MOE_TRY(need_ptr(X, "X"));
    MOE_TRY(need_ptr(W_r, "W_r"));
    MOE_TRY(opt_ptr(bias, "bias"));
  }
  MOE_TRY(check_ws(dims, MOE_OP_ROUTE, ws, ws_bytes));
  return do_route(dims, X, W_r, bias, logits, plan, ws, static_cast<hipStream_t>(stream));
}

size_t moe_route_noalloc_max_bytes(void) { return kRouteScratchBytes; }

moe_status moe_route_noalloc(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                             float* logits, const moe_plan* plan, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(logits, "logits"));
  if (X) {
    MOE_TRY(need_ptr(X, "X"));
    MOE_TRY(need_ptr(W_r, "W_r"));
    MOE_TRY(opt_ptr(bias, "bias"));
  }
  const size_t need = ws_bytes_for(dims, MOE_OP_ROUTE);
  if (need > kRouteScratchBytes)
    return fail(MOE_EWORKSPACE, "routing needs %zu bytes of workspace, more than the %zu of the static buffer",
                need, kRouteScratchBytes);
  void* ws = nullptr;
  MOE_TRY(route_scratch(&ws));
  return do_route(dims, X, W_r, bias, logits, plan, ws, static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_dims* dims, const moe_plan* plan, const void* X, void* X_perm,
                       void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(X, "X"));
  MOE_TRY(need_ptr(X_perm, "X_perm"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_STAGE(MOE_STAGE_PERMUTE, st, launch_permute(shape_of(dims), plan_ptrs(plan), X, X_perm, st), "permute");
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_dims* dims, const moe_plan* plan, const void* A_in,
                           int gathered, const void* W_gate, const void* W_up,
                           const void* W_down, void* H_cache, void* Y_perm, void* ws,
                           size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(A_in, gathered ? "X" : "X_perm"));
  MOE_TRY(need_ptr(W_gate, "W_gate"));
  MOE_TRY(need_ptr(W_up, "W_up"));
  MOE_TRY(need_ptr(W_down, "W_down"));
  MOE_TRY(opt_ptr(H_cache, "H_cache"));
  MOE_TRY(need_ptr(Y_perm, "Y_perm"));
  MOE_TRY(check_ws(dims, MOE_OP_FFN, ws, ws_bytes));
  Carve c(ws);
  const FfnWs w = carve_ffn(c, dims);
  return do_ffn(dims, plan, A_in, gathered != 0, W_gate, W_up, W_down, H_cache, Y_perm, w,
                static_cast<hipStream_t>(stream));
}

moe_status moe_combine(const moe_dims* dims, const moe_plan* plan, const void* Y_perm,
                       int weighted, void* out, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(Y_perm, "Y_perm"));
  MOE_TRY(need_ptr(out, "out"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_STAGE(MOE_STAGE_COMBINE, st, launch_combine(shape_of(dims), plan_ptrs(plan), Y_perm, weighted != 0, out, st),
            "combine");
  return MOE_OK;
}

moe_status moe_quantize_fp8(int64_t rows, int64_t K, int dtype, const void* src, uint8_t* codes,
                            float* scales, void* stream) {
  if (rows < 0 || rows > ((int64_t)1 << 31)) return fail(MOE_EINVAL, "rows=%lld out of range", (long long)rows);
  if (K < 8 || K > 65536 || K % 8) return fail(MOE_EINVAL, "K=%lld must be a multiple of 8 in [8, 65536]", (long long)K);
  if (dtype != MOE_BF16 && dtype != MOE_F32) return fail(MOE_ENOTSUP, "dtype %d not supported", dtype);
  if (rows == 0) return MOE_OK;
  MOE_TRY(need_ptr(src, "src"));
  MOE_TRY(need_ptr(codes, "codes"));
  MOE_TRY(need_ptr(scales, "scales"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_STAGE(MOE_STAGE_FP8_QUANT, st, launch_quant_fp8(src, dtype == MOE_BF16, rows, K, nullptr, codes, scales, st),
            "fp8 quantisation");
  return MOE_OK;
}

moe_status moe_grouped_ffn_fp8(const moe_dims* dims, const moe_plan* plan, const uint8_t* Xq,
                               const float* sx, const uint8_t* Wg_q, const float* sg,
                               const uint8_t* Wu_q, const float* su, const uint8_t* Wd_q,
                               const float* sd, void* act, uint8_t* act_q, float* sact,
                               void* Y_perm, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  if (dims->dtype != MOE_BF16) return fail(MOE_ENOTSUP, "moe_grouped_ffn_fp8 needs dtype MOE_BF16");
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(Xq, "Xq"));
  MOE_TRY(need_ptr(sx, "sx"));
  MOE_TRY(need_ptr(Wg_q, "Wg_q"));
  MOE_TRY(need_ptr(sg, "sg"));
  MOE_TRY(need_ptr(Wu_q, "Wu_q"));
  MOE_TRY(need_ptr(su, "su"));
  MOE_TRY(need_ptr(Wd_q, "Wd_q"));
  MOE_TRY(need_ptr(sd, "sd"));
  MOE_TRY(need_ptr(act, "act"));
  MOE_TRY(need_ptr(act_q, "act_q"));
  MOE_TRY(need_ptr(sact, "sact"));
  MOE_TRY(need_ptr(Y_perm, "Y_perm"));
  MOE_TRY(check_ws(dims, MOE_OP_FFN_FP8, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Shape s = shape_of(dims);
  const PlanPtrs p = plan_ptrs(plan);
  int32_t* mtile_off = static_cast<int32_t*>(ws);
  MOE_STAGE(MOE_STAGE_TILES, st, launch_tile_offsets(p.counts, dims->E, mtile_off, nullptr, st), "tile offsets");
  MOE_STAGE(MOE_STAGE_FP8_UP, st, launch_up_fp8(s, p, mtile_off, Xq, sx, Wg_q, sg, Wu_q, su, act, st),
            "fp8 gate/up GEMM");
  MOE_STAGE(MOE_STAGE_FP8_QUANT, st, launch_quant_fp8(act, true, s.R_max, dims->n, p.meta, act_q, sact, st),
            "fp8 activation quantisation");
  MOE_STAGE(MOE_STAGE_FP8_DOWN, st, launch_down_fp8(s, p, mtile_off, act_q, sact, Wd_q, sd, Y_perm, st),
            "fp8 down GEMM");
  return MOE_OK;
}

moe_status moe_decode(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                      const void* W_gate, const void* W_up, const void* W_down, float* logits,
                      int32_t* topk_idx, float* topk_w, void* out, void* ws, size_t ws_bytes,
                      void* stream) {
  MOE_TRY(check_dims(dims));
  if (dims->round_mode != MOE_ROUND_NONE)
    return fail(MOE_ENOTSUP, "moe_decode routes with plain top-K (round_mode must be NONE)");
  if (dims->T > 1024) return fail(MOE_ENOTSUP, "moe_decode handles T <= 1024 (got %lld)", (long long)dims->T);
  MOE_TRY(need_ptr(X, "X"));
  MOE_TRY(need_ptr(W_r, "W_r"));
  MOE_TRY(opt_ptr(bias, "bias"));
  MOE_TRY(need_ptr(W_gate, "W_gate"));
  MOE_TRY(need_ptr(W_up, "W_up"));
  MOE_TRY(need_ptr(W_down, "W_down"));
  MOE_TRY(need_ptr(logits, "logits"));
  MOE_TRY(need_ptr(topk_idx, "topk_idx"));
  MOE_TRY(need_ptr(topk_w, "topk_w"));
  MOE_TRY(need_ptr(out, "out"));
  MOE_TRY(check_ws(dims, MOE_OP_DECODE, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_STAGE(MOE_STAGE_DECODE, st,
            launch_decode(shape_of(dims), X, W_r, bias, W_gate, W_up, W_down, logits, topk_idx,
                          topk_w, out, ws, st),
            "decode");
  return MOE_OK;
}

int64_t moe_mx_scale_bytes(int64_t rows, int64_t K) { return rows >= 0 && K > 0 ? mx_scale_bytes(rows, K) : 0; }

moe_status moe_quantize_mx(int64_t rows, int64_t K, int dtype, int fmt, const void* src, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  if (rows < 0 || rows > ((int64_t)1 << 31)) return fail(MOE_EINVAL, "rows=%lld out of range", (long long)rows);
  if (K < 64 || K > 65536 || K % 64) return fail(MOE_EINVAL, "K=%lld must be a multiple of 64 in [64, 65536]", (long long)K);
  if (dtype != MOE_BF16 && dtype != MOE_F32) return fail(MOE_ENOTSUP, "dtype %d not supported", dtype);
  if (fmt != MOE_FP8_E4M3 && fmt != MOE_FP8_E5M2) return fail(MOE_EINVAL, "fp8 format %d invalid", fmt);
  if (rows == 0) return MOE_OK;
  MOE_TRY(need_ptr(src, "src"));
  MOE_TRY(need_ptr(codes, "codes"));
  MOE_TRY(need_ptr(scales, "scales"));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_STAGE(MOE_STAGE_FP8_QUANT, st, launch_quant_mx(src, dtype == MOE_BF16, fmt, rows, K, codes, scales, st),
            "block-scaled fp8 quantisation");
  return MOE_OK;
}

moe_status moe_grouped_ffn_mx(const moe_dims* dims, const moe_plan* plan, int fmt, const uint8_t* Xq,
                              const uint8_t* sx, const uint8_t* Wg_q, const uint8_t* sg, const uint8_t* Wu_q,
                              const uint8_t* su, const uint8_t* Wd_q, const uint8_t* sd, void* act,
                              uint8_t* act_q, uint8_t* sact, void* Y_perm, void* ws, size_t ws_bytes,
                              void* stream) {
  MOE_TRY(check_dims(dims));
  if (dims->dtype != MOE_BF16) return fail(MOE_ENOTSUP, "moe_grouped_ffn_mx needs dtype MOE_BF16");
  if (fmt != MOE_FP8_E4M3 && fmt != MOE_FP8_E5M2) return fail(MOE_EINVAL, "fp8 format %d invalid", fmt);
  if (dims->T * dims->d >= ((int64_t)1 << 32))
    return fail(MOE_ENOTSUP, "moe_grouped_ffn_mx needs T * d < 2^32 (T=%lld, d=%lld)", (long long)dims->T,
                (long long)dims->d);
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(Xq, "Xq"));
  MOE_TRY(need_ptr(sx, "sx"));
  MOE_TRY(need_ptr(Wg_q, "Wg_q"));
  MOE_TRY(need_ptr(sg, "sg"));
  MOE_TRY(need_ptr(Wu_q, "Wu_q"));
  MOE_TRY(need_ptr(su, "su"));
  MOE_TRY(need_ptr(Wd_q, "Wd_q"));
  MOE_TRY(need_ptr(sd, "sd"));
  MOE_TRY(opt_ptr(act, "act"));
  MOE_TRY(need_ptr(act_q, "act_q"));
  MOE_TRY(need_ptr(sact, "sact"));
  MOE_TRY(need_ptr(Y_perm, "Y_perm"));
  MOE_TRY(check_ws(dims, MOE_OP_FFN_MX, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Shape s = shape_of(dims);
  const PlanPtrs p = plan_ptrs(plan);
  Carve c(ws);
  int32_t* mtile_off = static_cast<int32_t*>(c.take((size_t)tile_table_ints(dims->E) * 4));
  uint8_t* sxp = static_cast<uint8_t*>(c.take((size_t)mx_scale_bytes(s.R_max, dims->d)));
  MOE_STAGE(MOE_STAGE_TILES, st, launch_tile_offsets(p.counts, dims->E, mtile_off, nullptr, st), "tile offsets");
  MOE_STAGE(MOE_STAGE_FP8_QUANT, st, launch_gather_mx_scales(s, p, sx, sxp, st), "token scale gather");
  MOE_STAGE(MOE_STAGE_FP8_UP, st,
            launch_up_mx(s, p, mtile_off, fmt, Xq, sxp, Wg_q, sg, Wu_q, su, act, act_q, sact, st),
            "block-scaled fp8 gate/up GEMM");
  MOE_STAGE(MOE_STAGE_FP8_DOWN, st, launch_down_mx(s, p, mtile_off, fmt, act_q, sact, Wd_q, sd, Y_perm, st),
            "block-scaled fp8 down GEMM");
  return MOE_OK;
}

moe_status moe_decode_status(void* stream) {
  int failed = 0;
  MOE_HIP(decode_read_status(static_cast<hipStream_t>(stream), &failed), "moe_decode_status");
  if (failed)
    return fail(MOE_EHIP, "moe_decode: a workgroup gave up waiting at a grid barrier; the outputs of "
                          "that call are invalid");
  return MOE_OK;
}

long long moe_decode_set_spin_limit(long long limit) {
  if (limit < 0) {
    fail(MOE_EINVAL, "spin limit %lld < 0", limit);
    return -1;
  }
  return decode_set_spin_limit(limit);
}

moe_status moe_forward(const moe_dims* dims, const void* X, const void* W_r, const float* bias,
                       const void* W_gate, const void* W_up, const void* W_down, float* logits,
                       const moe_plan* plan, void* H_cache, void* out, void* ws, size_t ws_bytes,
                       void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(X, "X"));
  MOE_TRY(need_ptr(W_r, "W_r"));
  MOE_TRY(opt_ptr(bias, "bias"));
  MOE_TRY(need_ptr(W_gate, "W_gate"));
  MOE_TRY(need_ptr(W_up, "W_up"));
  MOE_TRY(need_ptr(W_down, "W_down"));
  MOE_TRY(need_ptr(logits, "logits"));
  MOE_TRY(opt_ptr(H_cache, "H_cache"));
  MOE_TRY(need_ptr(out, "out"));
  MOE_TRY(check_ws(dims, MOE_OP_FORWARD, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  MOE_TRY(do_route(dims, X, W_r, bias, logits, plan, ws, st));
  Carve c(ws);
  const FfnWs w = carve_ffn(c, dims);
  void* Y = c.take((size_t)max_rows(dims) * dims->d * esize(dims));
  MOE_TRY(do_ffn(dims, plan, X, true, W_gate, W_up, W_down, H_cache, Y, w, st));
  MOE_STAGE(MOE_STAGE_COMBINE, st, launch_combine(shape_of(dims), plan_ptrs(plan), Y, true, out, st), "combine");
  return MOE_OK;
}

moe_status moe_backward(const moe_dims* dims, const void* dY, const void* X, const void* W_r,
                        const void* W_gate, const void* W_up, const void* W_down,
                        const moe_plan* plan, const void* H_cache, void* dX, void* dW_gate,
                        void* dW_up, void* dW_down, float* dS, float* dLogits, void* dW_r,
                        void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_dims(dims));
  MOE_TRY(check_plan(plan));
  MOE_TRY(need_ptr(dY, "dY"));
  MOE_TRY(need_ptr(X, "X"));
  MOE_TRY(opt_ptr(W_r, "W_r"));
  MOE_TRY(need_ptr(W_gate, "W_gate"));
  MOE_TRY(need_ptr(W_up, "W_up"));
  MOE_TRY(need_ptr(W_down, "W_down"));
  MOE_TRY(opt_ptr(H_cache, "H_cache"));
  MOE_TRY(need_ptr(dX, "dX"));
  MOE_TRY(need_ptr(dW_gate, "dW_gate"));
  MOE_TRY(need_ptr(dW_up, "dW_up"));
  MOE_TRY(need_ptr(dW_down, "dW_down"));
  MOE_TRY(need_ptr(dS, "dS"));
  MOE_TRY(need_ptr(dLogits, "dLogits"));
  MOE_TRY(opt_ptr(dW_r, "dW_r"));
  if (dW_r && !W_r) return fail(MOE_EINVAL, "dW_r requested without W_r");
  MOE_TRY(check_ws(dims, MOE_OP_BACKWARD, ws, ws_bytes));
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Shape s = shape_of(dims);
  const PlanPtrs p = plan_ptrs(plan);
  Carve c(ws);
  const BwdWs w = carve_bwd(c, dims);
  MOE_STAGE(MOE_STAGE_TILES, st, launch_tile_offsets(p.counts, dims->E, w.mtile_off, w.order, st),
            "tile offsets and expert order");
  const void* H = H_cache;
  if (!H) {  // recompute [G | U] from X; the SwiGLU output goes to wA, which dAct overwrites
    MOE_STAGE(MOE_STAGE_UP_GEMM, st, launch_up_gemm(s, p, w.mtile_off, X, true, W_gate, W_up, w.wA, w.H, st),
              "recompute GEMM");
    H = w.H;
  }
  MOE_STAGE(MOE_STAGE_DACT_GEMM, st,
            launch_dact_gemm(s, p, w.mtile_off, dY, W_down, H, w.dH, w.wA, w.dS_part, st), "dAct GEMM");
  MOE_STAGE(MOE_STAGE_DW_DOWN_GEMM, st, launch_dw_down_gemm(s, p, w.order, dY, w.wA, dW_down, st), "dW_down GEMM");
  MOE_STAGE(MOE_STAGE_DW_GU_GEMM, st, launch_dw_gu_gemm(s, p, w.order, w.dH, X, dW_gate, dW_up, st),
            "dW_gate/up GEMM");
  MOE_STAGE(MOE_STAGE_DX_GEMM, st, launch_dx_gemm(s, p, w.mtile_off, w.dH, W_gate, W_up, w.dX_perm, st),
            "dX GEMM");
  MOE_STAGE(MOE_STAGE_ROUTER_BWD, st,
            launch_router_bwd(s, p, w.dS_part, dact_ntiles(dims->n), w.dX_perm, W_r, dS, dLogits,
                              dW_r ? w.dLop : nullptr, e_pad(dims->E), dX, st),
            "router backward");
  if (dW_r)
    MOE_STAGE(MOE_STAGE_DWR_GEMM, st, launch_dwr_gemm(s, w.dLop, e_pad(dims->E), X, dW_r, w.dwr, st),
              "dW_r GEMM");
  return MOE_OK;
}

int moe_timing_enable(int on) {
  if (on) {
    if (!g_timing.created) {
      for (int i = 0; i < kTimingSlots; ++i) {
        if (hipEventCreate(&g_timing.ev0[i]) != hipSuccess || hipEventCreate(&g_timing.ev1[i]) != hipSuccess)
          return fail(MOE_EHIP, "hipEventCreate failed");
      }
      g_timing.created = true;
    }
    g_timing.used = 0;
    g_timing.on = true;
    return MOE_OK;
  }
  g_timing.on = false;
  hipError_t first = hipSuccess;
  if (g_timing.created) {
    for (int i = 0; i < g_timing.used; ++i) {
      const hipError_t e = hipEventSynchronize(g_timing.ev1[i]);
      if (first == hipSuccess) first = e;
    }
    for (int i = 0; i < kTimingSlots; ++i) {
      const hipError_t e0 = hipEventDestroy(g_timing.ev0[i]);
      const hipError_t e1 = hipEventDestroy(g_timing.ev1[i]);
      if (first == hipSuccess) first = e0 != hipSuccess ? e0 : e1;
    }
    g_timing.created = false;
  }
  g_timing.used = 0;
  return hip_status(first, "moe_timing_enable(0)");
}

int moe_timing_read(int stage, float* ms, int max) {
  if (stage < 0 || stage >= MOE_STAGE_COUNT) return fail(MOE_EINVAL, "unknown stage %d", stage);
  if (!ms && max > 0) return fail(MOE_EINVAL, "ms is NULL");
  int n = 0;
  for (int i = 0; i < g_timing.used && n < max; ++i) {
    if (g_timing.stage[i] != stage) continue;
    hipError_t e = hipEventSynchronize(g_timing.ev1[i]);
    float t = 0.0f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, g_timing.ev0[i], g_timing.ev1[i]);
    if (e != hipSuccess) return hip_status(e, "moe_timing_read");
    ms[n++] = t;
  }
  return n;
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_ENOTSUP: return "MOE_ENOTSUP: unsupported shape or dtype";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: HIP runtime error";
    default: return "unknown moe_status";
  }
}

const char* moe_last_error(void) { return g_err.c_str(); }

const char* moe_version(void) { return "moe_mi355x 0.1 (gfx950)"; }

}  // extern "C"

"""Thin ctypes binding of libmoe_mi355x.so (include/moe.h).

Argument marshalling only: torch tensors become device pointers, the current torch stream
becomes the hipStream_t, and non-zero status codes become ``MoEError``.  Every computation runs
in the library's HIP kernels; if the library is missing, the first call raises.
The functions keep the C names: ``moe_route``, ``moe_permute``, ``moe_grouped_ffn``,
``moe_combine``, ``moe_forward``, ``moe_backward``, ``moe_decode``, ``moe_quantize_fp8``,
``moe_grouped_ffn_fp8``, ``moe_quantize_mx``, ``moe_grouped_ffn_mx`` (plus sizing helpers).
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_F32, MOE_BF16 = 0, 1
ROUND_NONE, ROUND_NEAREST, ROUND_UP, ROUND_DOWN, ROUND_STOCHASTIC = 0, 1, 2, 3, 4
OP_ROUTE, OP_PERMUTE, OP_FFN, OP_COMBINE, OP_FORWARD, OP_BACKWARD, OP_DECODE, OP_FFN_FP8, OP_FFN_MX = range(9)
FP8_E4M3, FP8_E5M2 = 0, 1
STATUS = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_ENOTSUP", -3: "MOE_EWORKSPACE", -4: "MOE_EHIP"}

EXPORTS = ["moe_max_rows", "moe_workspace_bytes", "moe_route", "moe_permute", "moe_grouped_ffn",
           "moe_combine", "moe_forward", "moe_backward", "moe_decode", "moe_decode_status",
           "moe_route_noalloc", "moe_route_noalloc_max_bytes", "moe_mx_scale_bytes", "moe_quantize_mx",
           "moe_grouped_ffn_mx",
           "moe_decode_set_spin_limit", "moe_quantize_fp8",
           "moe_grouped_ffn_fp8", "moe_status_string", "moe_last_error",
           "moe_version", "moe_timing_enable", "moe_timing_read"]
STAGES = ["router_gemm", "route", "tiles", "up_gemm", "down_gemm", "permute", "combine", "dact_gemm",
          "dw_down_gemm", "dw_gu_gemm", "dx_gemm", "router_bwd", "dwr_gemm", "decode", "fp8_quant",
          "fp8_up_gemm", "fp8_down_gemm"]


class MoEError(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s: %s" % (STATUS.get(status, status), message))
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int64), ("n", ctypes.c_int64),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("round_mode", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("flags", ctypes.c_int32), ("round_rand", ctypes.c_void_p)]


PLAN_FIELDS = ["topk_idx", "topk_w", "counts", "expert_off", "row_token", "row_w", "tok_off",
               "tok_row", "meta"]


class PlanStruct(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in PLAN_FIELDS]


_lib = None


def lib():
    """The loaded library (loaded once; raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("%s is missing: build it with `python -m mixture_experts_layer_lds_amd.build`"
                               % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        pd = ctypes.POINTER(Dims)
        pp = ctypes.POINTER(PlanStruct)
        L.moe_max_rows.argtypes, L.moe_max_rows.restype = [pd], ctypes.c_int64
        L.moe_workspace_bytes.argtypes, L.moe_workspace_bytes.restype = [pd, ctypes.c_int], sz
        L.moe_route.argtypes = [pd, vp, vp, vp, vp, pp, vp, sz, vp]
        L.moe_route_noalloc.argtypes = [pd, vp, vp, vp, vp, pp, vp]
        L.moe_route_noalloc_max_bytes.argtypes, L.moe_route_noalloc_max_bytes.restype = [], sz
        L.moe_permute.argtypes = [pd, pp, vp, vp, vp]
        L.moe_grouped_ffn.argtypes = [pd, pp, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.argtypes = [pd, pp, vp, ctypes.c_int, vp, vp]
        L.moe_forward.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, sz, vp]
        L.moe_backward.argtypes = [pd, vp, vp, vp, vp, vp, vp, pp, vp, vp, vp, vp, vp, vp, vp, vp,
                                   vp, sz, vp]
        L.moe_decode.argtypes = [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_decode_status.argtypes, L.moe_decode_status.restype = [vp], st
        L.moe_decode_set_spin_limit.argtypes = [ctypes.c_longlong]
        L.moe_decode_set_spin_limit.restype = ctypes.c_longlong
        L.moe_quantize_fp8.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, vp, vp, vp, vp]
        L.moe_grouped_ffn_fp8.argtypes = [pd, pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_mx_scale_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64]
        L.moe_mx_scale_bytes.restype = ctypes.c_int64
        L.moe_quantize_mx.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp]
        L.moe_grouped_ffn_mx.argtypes = [pd, pp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                         sz, vp]
        for f in ("moe_route", "moe_route_noalloc", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_forward",
                  "moe_backward", "moe_decode", "moe_quantize_fp8", "moe_grouped_ffn_fp8", "moe_quantize_mx",
                  "moe_grouped_ffn_mx"):
            getattr(L, f).restype = st
        L.moe_status_string.argtypes, L.moe_status_string.restype = [ctypes.c_int], ctypes.c_char_p
        L.moe_last_error.argtypes, L.moe_last_error.restype = [], ctypes.c_char_p
        L.moe_version.argtypes, L.moe_version.restype = [], ctypes.c_char_p
        L.moe_timing_enable.argtypes, L.moe_timing_enable.restype = [ctypes.c_int], ctypes.c_int
        L.moe_timing_read.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.moe_timing_read.restype = ctypes.c_int
        _lib = L
    return _lib


def make_dims(T, d, n, E, K, dtype="bf16", round_mode=ROUND_NONE, tile_m=128, round_rand=None):
    """Layer shape; ``round_rand`` is the [E] int32/uint32 device tensor of random words that
    stochastic token rounding reads (the caller keeps it alive while the dims are used)."""
    dt = {"bf16": MOE_BF16, "f32": MOE_F32, torch.bfloat16: MOE_BF16, torch.float32: MOE_F32}[dtype]
    return Dims(int(T), int(d), int(n), int(E), int(K), dt, int(round_mode), int(tile_m), 0,
                _p(round_rand))


def torch_dtype(dims):
    return torch.bfloat16 if dims.dtype == MOE_BF16 else torch.float32


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _check(status):
    if status != 0:
        raise MoEError(status, lib().moe_last_error().decode())


def moe_max_rows(dims):
    r = lib().moe_max_rows(ctypes.byref(dims))
    if r == 0:
        raise MoEError(-1, lib().moe_last_error().decode())
    return r


def moe_workspace_bytes(dims, op):
    return lib().moe_workspace_bytes(ctypes.byref(dims), op)


class Plan:
    """Caller-owned routing plan: the device arrays of ``moe_plan`` with their ctypes view."""

    def __init__(self, dims, device="cuda"):
        T, E, K = dims.T, dims.E, dims.K
        R = moe_max_rows(dims)
        i32, f32 = torch.int32, torch.float32
        self.R_max = R
        self.topk_idx = torch.empty(T * K, dtype=i32, device=device)
        self.topk_w = torch.empty(T * K, dtype=f32, device=device)
        self.counts = torch.empty(E, dtype=i32, device=device)
        self.expert_off = torch.empty(E + 1, dtype=i32, device=device)
        self.row_token = torch.empty(R, dtype=i32, device=device)
        self.row_w = torch.empty(R, dtype=f32, device=device)
        self.tok_off = torch.empty(T + 1, dtype=i32, device=device)
        self.tok_row = torch.empty(R, dtype=i32, device=device)
        self.meta = torch.zeros(16, dtype=i32, device=device)
        self.struct = PlanStruct(*[getattr(self, f).data_ptr() for f in PLAN_FIELDS])

    def ref(self):
        return ctypes.byref(self.struct)

    def to_host(self):
        """numpy copies of the plan arrays, trimmed to the actual row count R."""
        R = int(self.meta[0].item())
        out = {f: getattr(self, f).cpu().numpy() for f in PLAN_FIELDS}
        for f in ("row_token", "row_w", "tok_row"):
            out[f] = out[f][:R]
        out["R"] = R
        return out


def workspace(dims, op, device="cuda"):
    nbytes = moe_workspace_bytes(dims, op)
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device), nbytes


def moe_route(dims, X, W_r, bias, logits, plan, ws, ws_bytes, stream=None):
    _check(lib().moe_route(ctypes.byref(dims), _p(X), _p(W_r), _p(bias), _p(logits), plan.ref(),
                           _p(ws), ws_bytes, _stream(stream)))


def moe_route_noalloc(dims, X, W_r, bias, logits, plan, stream=None):
    """moe_route with the library's static routing buffer as workspace (no allocation)."""
    _check(lib().moe_route_noalloc(ctypes.byref(dims), _p(X), _p(W_r), _p(bias), _p(logits), plan.ref(),
                                   _stream(stream)))


def moe_route_noalloc_max_bytes():
    return lib().moe_route_noalloc_max_bytes()


def moe_permute(dims, plan, X, X_perm, stream=None):
    _check(lib().moe_permute(ctypes.byref(dims), plan.ref(), _p(X), _p(X_perm), _stream(stream)))


def moe_grouped_ffn(dims, plan, A_in, gathered, W_gate, W_up, W_down, H_cache, Y_perm, ws, ws_bytes,
                    stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(dims), plan.ref(), _p(A_in), int(bool(gathered)),
                                 _p(W_gate), _p(W_up), _p(W_down), _p(H_cache), _p(Y_perm), _p(ws),
                                 ws_bytes, _stream(stream)))


def moe_combine(dims, plan, Y_perm, weighted, out, stream=None):
    _check(lib().moe_combine(ctypes.byref(dims), plan.ref(), _p(Y_perm), int(bool(weighted)), _p(out),
                             _stream(stream)))


def moe_forward(dims, X, W_r, bias, W_gate, W_up, W_down, logits, plan, H_cache, out, ws, ws_bytes,
                stream=None):
    _check(lib().moe_forward(ctypes.byref(dims), _p(X), _p(W_r), _p(bias), _p(W_gate), _p(W_up),
                             _p(W_down), _p(logits), plan.ref(), _p(H_cache), _p(out), _p(ws), ws_bytes,
                             _stream(stream)))


def moe_decode(dims, X, W_r, bias, W_gate, W_up, W_down, logits, topk_idx, topk_w, out, ws, ws_bytes,
               stream=None):
    _check(lib().moe_decode(ctypes.byref(dims), _p(X), _p(W_r), _p(bias), _p(W_gate), _p(W_up),
                            _p(W_down), _p(logits), _p(topk_idx), _p(topk_w), _p(out), _p(ws), ws_bytes,
                            _stream(stream)))


def moe_decode_status(stream=None):
    """Raises MoEError(MOE_EHIP) if a moe_decode kernel on the current device gave up at a grid
    barrier since the last check (waits for the stream first); clears the device's status word."""
    _check(lib().moe_decode_status(_stream(stream)))


def moe_decode_set_spin_limit(limit):
    """Polls before a moe_decode grid barrier gives up (later launches); returns the previous limit."""
    prev = lib().moe_decode_set_spin_limit(int(limit))
    if prev < 0:
        raise MoEError(-1, lib().moe_last_error().decode())
    return prev


def moe_quantize_fp8(src, codes, scales, stream=None):
    """Per-row E4M3 codes and power-of-two scales of a 2-D bf16 / fp32 tensor (rows x K)."""
    rows, K = src.shape[0], src.shape[-1]
    dtype = MOE_BF16 if src.dtype == torch.bfloat16 else MOE_F32
    _check(lib().moe_quantize_fp8(rows, K, dtype, _p(src), _p(codes), _p(scales), _stream(stream)))


def moe_grouped_ffn_fp8(dims, plan, Xq, sx, Wg_q, sg, Wu_q, su, Wd_q, sd, act, act_q, sact, Y_perm, ws,
                        ws_bytes, stream=None):
    _check(lib().moe_grouped_ffn_fp8(ctypes.byref(dims), plan.ref(), _p(Xq), _p(sx), _p(Wg_q), _p(sg),
                                     _p(Wu_q), _p(su), _p(Wd_q), _p(sd), _p(act), _p(act_q), _p(sact),
                                     _p(Y_perm), _p(ws), ws_bytes, _stream(stream)))


def moe_mx_scale_bytes(rows, K):
    return lib().moe_mx_scale_bytes(int(rows), int(K))


def moe_quantize_mx(src, fmt, codes, scales, stream=None):
    """Block-scaled FP8 codes and E8M0 scale bytes of a 2-D bf16 / fp32 tensor (rows x K)."""
    rows, K = src.shape[0], src.shape[-1]
    dtype = MOE_BF16 if src.dtype == torch.bfloat16 else MOE_F32
    _check(lib().moe_quantize_mx(rows, K, dtype, int(fmt), _p(src), _p(codes), _p(scales), _stream(stream)))


def moe_grouped_ffn_mx(dims, plan, fmt, Xq, sx, Wg_q, sg, Wu_q, su, Wd_q, sd, act, act_q, sact, Y_perm, ws, ws_bytes,
                       stream=None):
    _check(lib().moe_grouped_ffn_mx(ctypes.byref(dims), plan.ref(), int(fmt), _p(Xq), _p(sx), _p(Wg_q), _p(sg),
                                    _p(Wu_q), _p(su), _p(Wd_q), _p(sd), _p(act), _p(act_q), _p(sact), _p(Y_perm),
                                    _p(ws), ws_bytes, _stream(stream)))


def moe_backward(dims, dY, X, W_r, W_gate, W_up, W_down, plan, H_cache, dX, dW_gate, dW_up, dW_down,
                 dS, dLogits, dW_r, ws, ws_bytes, stream=None):
    _check(lib().moe_backward(ctypes.byref(dims), _p(dY), _p(X), _p(W_r), _p(W_gate), _p(W_up),
                              _p(W_down), plan.ref(), _p(H_cache), _p(dX), _p(dW_gate), _p(dW_up),
                              _p(dW_down), _p(dS), _p(dLogits), _p(dW_r), _p(ws), ws_bytes,
                              _stream(stream)))


def moe_timing_enable(on):
    _check(lib().moe_timing_enable(int(bool(on))))


def moe_timing_read(stage, max_n=4096):
    """Per-launch durations (ms) recorded for a stage (name or index) since timing was enabled."""
    idx = STAGES.index(stage) if isinstance(stage, str) else int(stage)
    buf = (ctypes.c_float * max_n)()
    n = lib().moe_timing_read(idx, buf, max_n)
    if n < 0:
        _check(n)
    return list(buf[:n])

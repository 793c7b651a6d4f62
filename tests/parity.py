"""Helpers for GPU-vs-oracle parity tests: run the HIP library through its C ABI on seeded
inputs, and compare with the float64 oracle fed the very same tensors.

Tolerances are the ones the layer is specified to: integer routing outputs bit-exact given the
same fp32 logits; every floating-point tensor y satisfies max|y - y_ref| <= tol * max|y_ref| with
tol = 1e-4 for fp32 layers and 2e-2 for bf16 layers.
"""
import numpy as np
import torch

import oracle
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl

TOL = {"f32": 1e-4, "bf16": 2e-2}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(y - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def assert_close(name, y, ref, tol):
    e = rel_err(y, ref)
    assert e <= tol, "%s: max|y-ref|/max|ref| = %.3e > %.1e" % (name, e, tol)
    return e


class LazyExperts:
    """W[e] -> float64 numpy of one expert's matrix, converted on demand (big layers)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return f64(self.t[e])

    def __len__(self):
        return self.t.shape[0]


def dims_of(cfg, round_rand=None):
    return B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype, cfg.round_mode, cfg.tile_m, round_rand)


def run_gpu(cfg, inputs=None, backward=None, cache_h=True, with_router_grad=True):
    """Forward (and backward) of one layer on cuda:0 through the C ABI.  Returns a dict of tensors."""
    dev = "cuda"
    inp = inputs if inputs is not None else wl.make_inputs(cfg, device=dev)
    backward = cfg.backward if backward is None else backward
    dims = dims_of(cfg, inp["round_rand"])
    dt = B.torch_dtype(dims)
    plan = B.Plan(dims, dev)
    R_max = plan.R_max
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev)
    H = torch.empty(R_max, 2 * cfg.n, dtype=dt, device=dev) if cache_h or backward else None
    out = torch.empty(cfg.T, cfg.d, dtype=dt, device=dev)
    ws, nb = B.workspace(dims, B.OP_FORWARD, dev)
    B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                  logits, plan, H, out, ws, nb)
    res = dict(inputs=inp, dims=dims, plan=plan, logits=logits, H=H, out=out)
    if backward:
        dY = inp["dY"]
        g = dict(dX=torch.empty_like(inp["X"]), dW_gate=torch.empty_like(inp["W_gate"]),
                 dW_up=torch.empty_like(inp["W_up"]), dW_down=torch.empty_like(inp["W_down"]),
                 dS=torch.empty(R_max, dtype=torch.float32, device=dev),
                 dLogits=torch.empty(cfg.T, cfg.E, dtype=torch.float32, device=dev),
                 dW_r=torch.empty_like(inp["W_r"]) if with_router_grad else None)
        wsb, nbb = B.workspace(dims, B.OP_BACKWARD, dev)
        B.moe_backward(dims, dY, inp["X"], inp["W_r"] if with_router_grad else None, inp["W_gate"],
                       inp["W_up"], inp["W_down"], plan, H if cache_h else None, g["dX"], g["dW_gate"],
                       g["dW_up"], g["dW_down"], g["dS"], g["dLogits"], g["dW_r"], wsb, nbb)
        res.update(g)
    torch.cuda.synchronize()
    return res


def run_grouped_ffn(cfg, res):
    """moe_grouped_ffn on gathered rows with the plan of ``res`` (the kernels moe_forward runs):
    returns (H, Y_perm) as device tensors, so that Y_perm rows, which moe_forward keeps in its
    workspace, can be compared."""
    dims, plan, inp = res["dims"], res["plan"], res["inputs"]
    dt = B.torch_dtype(dims)
    H = torch.empty(plan.R_max, 2 * cfg.n, dtype=dt, device="cuda")
    Y = torch.empty(plan.R_max, cfg.d, dtype=dt, device="cuda")
    ws, nb = B.workspace(dims, B.OP_FFN, "cuda")
    B.moe_grouped_ffn(dims, plan, inp["X"], 1, inp["W_gate"], inp["W_up"], inp["W_down"], H, Y, ws, nb)
    torch.cuda.synchronize()
    del ws
    return H, Y


def check_routing(cfg, res, L=None, round_rand=None):
    """Routing outputs bit-exact against the oracle run on the GPU's fp32 logits (and, for
    stochastic token rounding, the same random words)."""
    if L is None:
        L = f64(res["logits"])
    if round_rand is None and "inputs" in res:
        round_rand = res["inputs"]["round_rand"]
    words = wl.round_rand_words(round_rand) if round_rand is not None else None
    ref = oracle.build_plan(L, cfg.K, round_mode=cfg.round_mode, tile_m=cfg.tile_m, round_rand=words)
    got = res["plan"].to_host()
    T, K = cfg.T, cfg.K
    assert np.array_equal(got["topk_idx"].reshape(T, K), ref["topk_idx"]), "topk_idx"
    assert np.array_equal(got["counts"], ref["counts"]), "counts"
    assert np.array_equal(got["expert_off"], ref["expert_off"]), "expert_off"
    assert got["R"] == int(ref["expert_off"][-1])
    assert np.array_equal(got["row_token"], ref["row_token"]), "row_token"
    assert np.array_equal(got["tok_off"], ref["tok_off"]), "tok_off"
    assert np.array_equal(got["tok_row"], ref["tok_row"]), "tok_row"
    tol = TOL[cfg.dtype]
    assert_close("topk_w", got["topk_w"].reshape(T, K), ref["topk_w"], tol)
    assert_close("row_w", got["row_w"], ref["row_w"], tol)
    return ref


def check_forward(cfg, res, ref_plan):
    inp = res["inputs"]
    tol = TOL[cfg.dtype]
    X = f64(inp["X"])
    L_ref = oracle.router_logits(X, f64(inp["W_r"]), None if inp["bias"] is None else f64(inp["bias"]))
    errs = dict(logits=assert_close("logits", f64(res["logits"]), L_ref, tol))
    fw = oracle.layer_forward(X, f64(inp["W_gate"]), f64(inp["W_up"]), f64(inp["W_down"]), ref_plan)
    errs["out"] = assert_close("out", f64(res["out"]), fw["out"], tol)
    R = int(ref_plan["expert_off"][-1])
    if res["H"] is not None and R:
        errs["H"] = assert_close("H", f64(res["H"][:R]), fw["H"], tol)
    return errs, fw


def check_backward(cfg, res, ref_plan):
    inp = res["inputs"]
    tol = TOL[cfg.dtype]
    bw = oracle.layer_backward(f64(inp["dY"]), f64(inp["X"]), f64(inp["W_gate"]), f64(inp["W_up"]),
                               f64(inp["W_down"]), ref_plan,
                               W_r=f64(inp["W_r"]) if res.get("dW_r") is not None else None)
    E = cfg.E
    R = int(ref_plan["expert_off"][-1])
    errs = {}
    errs["dX"] = assert_close("dX", f64(res["dX"]), bw["dX"], tol)
    errs["dS"] = assert_close("dS", f64(res["dS"][:R]), bw["dS"], tol)
    errs["dLogits"] = assert_close("dLogits", f64(res["dLogits"]), bw["dLogits"], tol)
    for k in ("dW_gate", "dW_up", "dW_down"):
        ref = np.stack([bw[k][e] for e in range(E)])
        errs[k] = assert_close(k, f64(res[k]), ref, tol)
    if res.get("dW_r") is not None:
        errs["dW_r"] = assert_close("dW_r", f64(res["dW_r"]), bw["dW_r"], tol)
    return errs


def subset_plan(plan, tokens):
    """The routing plan restricted to the rows of `tokens` (same experts, same weights)."""
    tokens = np.asarray(sorted(set(int(t) for t in tokens)))
    keep = np.isin(plan["row_token"], tokens)
    rows = np.nonzero(keep)[0]
    E = len(plan["expert_off"]) - 1
    counts = np.bincount(plan["row_expert"][rows], minlength=E)
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(counts)
    T = len(plan["tok_off"]) - 1
    sub = dict(expert_off=off, row_token=plan["row_token"][rows], row_expert=plan["row_expert"][rows],
               row_w=plan["row_w"][rows])
    # token-major CSR over the kept rows (rows of a token ascending in expert)
    newidx = -np.ones(len(plan["row_token"]), np.int64)
    newidx[rows] = np.arange(len(rows))
    tok_counts = np.zeros(T, np.int64)
    tok_rows = []
    for t in tokens:                                   # ascending token id
        rr = plan["tok_row"][plan["tok_off"][t]:plan["tok_off"][t + 1]]
        tok_rows.append(newidx[rr])
        tok_counts[t] = len(rr)
    tok_off = np.zeros(T + 1, np.int64)
    tok_off[1:] = np.cumsum(tok_counts)
    sub["tok_off"] = tok_off
    sub["tok_row"] = np.concatenate(tok_rows) if tok_rows else np.zeros(0, np.int64)
    return sub, rows


class ExpertSubset:
    """W[j] = W[experts[j]]: the weights of a plan compacted to the experts it uses."""

    def __init__(self, W, experts):
        self.W = W
        self.experts = experts

    def __getitem__(self, j):
        return self.W[int(self.experts[j])]

    def __len__(self):
        return len(self.experts)


def compact_plan(plan):
    """The plan renumbered to the experts that own rows (ascending id), so that the oracle's loops
    over experts visit only those.  Returns (compacted plan, the experts' original ids)."""
    used = np.unique(plan["row_expert"])
    new_of = {int(e): j for j, e in enumerate(used)}
    row_expert = np.array([new_of[int(e)] for e in plan["row_expert"]], np.int64)
    off = np.zeros(len(used) + 1, np.int64)
    off[1:] = np.cumsum(np.bincount(row_expert, minlength=len(used)))
    out = dict(plan)
    out.update(expert_off=off, row_expert=row_expert)
    return out, used

#!/usr/bin/env python3
"""Benchmark of the one-GPU MoE layer on MI355X: useful TFLOP/s of forward + backward.

Default workload: the fine-grained 7B-style layer (T=32768 tokens, d=1536, E=128 experts, top-8,
SwiGLU experts of width n=256, bf16), forward + backward, seeded synthetic inputs resident in HBM.
One step = moe_forward (router GEMM, routing, gathered gate/up GEMM with SwiGLU, down GEMM,
weighted combine) + moe_backward (dAct with SwiGLU backward and dS, dW_down, dW_gate/up, dX,
router backward with the dX gather-sum, router weight gradient).

Prints ONE JSON line.  "Useful" FLOPs count real (token, expert) rows only:
6 R d n forward + 12 R d n backward for the experts, plus 2 T d E (router forward) and
4 T d E (router backward).  The K timed steps run with the library's stage timing off; a second
pass of K steps records a hipEvent pair around each stage on the stream the library launches it
on, which gives the per-stage durations and the roofline of the dominant kernel.  Combine and
permute are also timed on their own with a 1 GiB write between reps that flushes the caches
(median and min).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME] [--no-cpu]
"""
import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_FP32_TFLOPS = 157.3      # MI355X dense fp32 MFMA (published)
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "MoE layer fwd+bwd useful TFLOPS and % bf16 MFMA peak, T=32768 fine-grained"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="fine_grained_7b")
    ap.add_argument("--round-mode", type=int, default=None,
                    help="override token rounding: 0 none, 1 nearest, 2 up, 3 down, 4 stochastic")
    ap.add_argument("--tile-m", type=int, default=None, help="override the token-rounding tile (with --round-mode)")
    ap.add_argument("--no-h-cache", action="store_true", help="backward recomputes [G|U] from X")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU baseline time budget")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--decode", type=int, default=0, metavar="T",
                    help="instead of the layer step, time moe_decode (single-launch forward) on T "
                         "tokens of --config, next to moe_forward on the same tokens")
    ap.add_argument("--fp8", action="store_true",
                    help="instead of the layer step, time the forward with FP8 expert GEMMs (moe_route, "
                         "moe_quantize_fp8 of X, moe_grouped_ffn_fp8, moe_combine) next to the bf16 moe_forward")
    ap.add_argument("--mx", choices=["e4m3", "e5m2"], default=None,
                    help="instead of the layer step, time the forward with block-scaled FP8 expert GEMMs (moe_route, "
                         "moe_quantize_mx of X, moe_grouped_ffn_mx, moe_combine) next to the bf16 moe_forward")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after warmup, run a plain 256 MiB copy kernel (torch neg on fp32) three times, "
                         "outside the timed region: the byte counters of a profiler run are scaled by it")
    return ap.parse_args()


def stage_flops(stage, R, T, d, n, E):
    """Algorithmic FLOPs of one launch of a GEMM stage (real rows only)."""
    return {
        "router_gemm": 2 * T * d * E,
        "up_gemm": 4 * R * d * n,
        "down_gemm": 2 * R * d * n,
        "dact_gemm": 2 * R * d * n,
        "dw_down_gemm": 2 * R * d * n,
        "dw_gu_gemm": 4 * R * d * n,
        "dx_gemm": 4 * R * d * n,
        "dwr_gemm": 2 * T * d * E,
    }.get(stage)


def stage_bytes(stage, R, T, d, n, E, es, K=None):
    """Algorithmic HBM bytes of one launch of a streaming stage.  Routing reads the fp32 logits
    and writes the plan: top-K ids and weights, expert-major rows (token, weight) and the
    token-major inverse (offsets, rows).  The router backward reads each row's dX_perm row, index,
    weight and dS partial, writes dS, the fp32 dLogits, the router weight gradient's dL operand
    and dX (the router weights it reads stay in the L2)."""
    K = K if K is not None else max(1, R // max(T, 1))
    return {
        "route": T * E * 4 + T * K * 8 + R * 12 + (T + 1) * 4,
        "permute": R * d * es + T * d * es + R * 4,
        "combine": R * d * es + T * d * es + R * 8 + (T + 1) * 4,
        "router_bwd": R * d * es + T * d * es + T * E * (4 + es) + R * 16 + (T + 1) * 4,
    }.get(stage)


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "traffic_counters.json")


def kernel_source_digest():
    """sha256 over the HIP/C++ sources of the library (file names and code, sorted), with comments
    and blank lines stripped, so that a record stays valid across edits of comments only."""
    import hashlib
    import re
    src = os.path.join(HERE, "mixture_experts_layer_lds_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(src)):
        if f.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(src, f), encoding="utf-8") as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
            h.update(f.encode())
            h.update("\n".join(l for l in lines if l.strip()).encode())
    return h.hexdigest()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` from the recorded FETCH_SIZE / WRITE_SIZE counter runs
    (already scaled by the copy-kernel calibration), or None when there is no record for this
    workload and stage or when any kernel source changed after the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_digest():
        return None
    ent = rec.get("workloads", {}).get(workload, {}).get(stage)
    return int(ent["hbm_bytes_per_launch"]) if ent else None


def stage_min_bytes(stage, R, T, d, n, E, es):
    """Compulsory HBM bytes of one launch of a GEMM stage: every operand read once and every
    result written once (the floor that `traffic` is compared against)."""
    Wb = E * d * n * es            # one expert weight matrix set [E, n, d] or [E, d, n]
    return {
        "router_gemm": T * d * es + E * d * es + T * E * 4,
        "up_gemm": T * d * es + 2 * Wb + R * n * es + R * 2 * n * es + R * 4,
        "down_gemm": R * n * es + Wb + R * d * es,
        "dact_gemm": T * d * es + Wb + R * 2 * n * es + R * 2 * n * es + R * n * es + R * 8,
        "dw_down_gemm": T * d * es + R * n * es + Wb,
        "dw_gu_gemm": R * 2 * n * es + T * d * es + 2 * Wb,
        "dx_gemm": R * 2 * n * es + 2 * Wb + R * d * es,
        "dwr_gemm": T * E * 4 + T * d * es + E * d * es,
    }.get(stage)


def memory_accounting(cfg, dims, R_max, backward, B):
    """Bytes the layer keeps from the forward to the backward, and the workspaces: with the H
    cache (H = [G|U], the plan and the logits) and with full recompute (the plan and the logits),
    against a layer that also keeps the gathered inputs, the SwiGLU output and the expert outputs
    (X_perm [R,d], A [R,n], Y [R,d] besides H)."""
    es = 2 if cfg.dtype == "bf16" else 4
    T, d, n, E, K = cfg.T, cfg.d, cfg.n, cfg.E, cfg.K
    plan = T * K * 8 + E * 8 + 4 + R_max * 12 + (T + 1) * 4 + 64
    logits = T * E * 4
    H = R_max * 2 * n * es
    conventional = plan + logits + H + R_max * d * es + R_max * n * es + R_max * d * es
    m = {"kept_with_h_cache": plan + logits + H, "kept_recompute": plan + logits,
         "kept_conventional": conventional,
         "forward_workspace": int(B.moe_workspace_bytes(dims, B.OP_FORWARD))}
    if backward:
        m["backward_workspace"] = int(B.moe_workspace_bytes(dims, B.OP_BACKWARD))
    return m


def cpu_baseline(cfg, inp, logits, budget_s):
    """The float64 oracle, as it stands, on a bounded sample of the same layer: whole experts'
    forward + backward, experts taken in a seeded order until the time budget is used."""
    import torch
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    L = logits.double().cpu().numpy()
    from mixture_experts_layer_lds_amd import workloads as wl
    plan = oracle.build_plan(L, cfg.K, round_mode=cfg.round_mode, tile_m=cfg.tile_m,
                             round_rand=wl.round_rand_words(inp["round_rand"]))
    X = inp["X"].double().cpu().numpy()
    dY = inp["dY"].double().cpu().numpy() if "dY" in inp else None

    class Lazy:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return self.t[e].double().cpu().numpy()

    Wg, Wu, Wd = Lazy(inp["W_gate"]), Lazy(inp["W_up"]), Lazy(inp["W_down"])
    order = np.random.default_rng(1234).permutation(cfg.E)
    rows = 0
    used = []
    t_total = 0.0
    for e in order:
        t0 = time.perf_counter()
        oracle.layer_forward(X, Wg, Wu, Wd, plan, experts=[int(e)])
        if dY is not None:
            oracle.layer_backward(dY, X, Wg, Wu, Wd, plan, experts=[int(e)])
        t_total += time.perf_counter() - t0
        rows += int(plan["counts"][e])
        used.append(int(e))
        if t_total >= budget_s:
            break
    mult = 18 if dY is not None else 6
    flops = mult * rows * cfg.d * cfg.n
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of %d experts (%d token rows), expert SwiGLU FFN %s in float64 numpy, %.1f s"
                      % (len(used), cfg.E, rows, "forward+backward" if dY is not None else "forward", t_total)}


def decode_bench(args):
    """moe_decode on T tokens of a layer shape: per-call latency, the HBM bytes it must move (the
    routed experts' weights once each, router weights, tokens in and out), and moe_forward on the
    same tokens for comparison."""
    import torch
    from mixture_experts_layer_lds_amd import binding as B
    from mixture_experts_layer_lds_amd import workloads as wl

    cfg = wl.BY_NAME[args.config].with_(T=args.decode, backward=False, round_mode=0)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=False)
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype)
    dt = B.torch_dtype(dims)
    es = 2 if cfg.dtype == "bf16" else 4
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    topk_idx = torch.empty(cfg.T, cfg.K, dtype=torch.int32, device="cuda")
    topk_w = torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda")
    out = torch.empty(cfg.T, cfg.d, dtype=dt, device="cuda")
    ws, nb = B.workspace(dims, B.OP_DECODE)
    plan = B.Plan(dims)
    of = torch.empty_like(out)
    wsf, nbf = B.workspace(dims, B.OP_FORWARD)

    def dec():
        B.moe_decode(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                     logits, topk_idx, topk_w, out, ws, nb)

    def fwd():
        B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                      logits, plan, None, of, wsf, nbf)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    ms_fwd = timed(fwd)
    B.moe_timing_enable(True)
    ms = timed(dec)
    kern = B.moe_timing_read("decode")
    B.moe_timing_enable(False)
    kern_ms = float(np.mean(kern[args.warmup:] if len(kern) > args.warmup else kern))
    used = np.unique(topk_idx.cpu().numpy())
    nbytes = (len(used) * 3 * cfg.n * cfg.d * es + cfg.E * cfg.d * es + 2 * cfg.T * cfg.d * es
              + cfg.T * cfg.E * 4 + cfg.T * cfg.K * 8)
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MoE decode layer forward, single launch (%s, T=%d)" % (cfg.name, cfg.T),
        "value": round(cfg.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded normal inputs and random-init weights)",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "n": cfg.n, "E": cfg.E, "K": cfg.K,
                   "experts_used": int(len(used)), "parallelism": "single GPU"},
        "roofline": {"kernel": "decode", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "avg_ms": round(kern_ms, 4), "algorithmic_bytes": int(nbytes)},
        "moe_forward_ms": round(ms_fwd, 4),
        "speedup_vs_moe_forward": round(ms_fwd / ms, 2),
    }
    print(json.dumps(res), flush=True)


def fp8_bench(args):
    """Forward layer with FP8 expert GEMMs on --config: routing as in bf16, X quantised each step,
    the experts' weights quantised once before timing (they are the stored model).  --fp8: per-row
    power-of-two scales, the activation quantised by a separate pass inside
    moe_grouped_ffn_fp8; --mx FMT: 32-element block scales applied by the MFMA, the activation
    quantised in the gate/up GEMM's epilogue.  Useful FLOPs as for the bf16 forward."""
    import torch
    from mixture_experts_layer_lds_amd import binding as B
    from mixture_experts_layer_lds_amd import workloads as wl

    cfg = wl.BY_NAME[args.config].with_(backward=False, round_mode=0)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=False)
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16", cfg.round_mode, cfg.tile_m,
                       inp["round_rand"])
    T, d, n, E = cfg.T, cfg.d, cfg.n, cfg.E
    plan = B.Plan(dims)
    R_max = plan.R_max
    u8 = dict(dtype=torch.uint8, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    mx = args.mx is not None
    fmt = {"e4m3": B.FP8_E4M3, "e5m2": B.FP8_E5M2}.get(args.mx)

    def quant(t, rows, K):
        c = torch.empty(rows, K, **u8)
        if mx:
            s_ = torch.empty(B.moe_mx_scale_bytes(rows, K), **u8)
            B.moe_quantize_mx(t.reshape(rows, K), fmt, c, s_)
        else:
            s_ = torch.empty(rows, **f32)
            B.moe_quantize_fp8(t.reshape(rows, K), c, s_)
        return c, s_

    Wgq, sg = quant(inp["W_gate"], E * n, d)
    Wuq, su = quant(inp["W_up"], E * n, d)
    Wdq, sd = quant(inp["W_down"], E * d, n)
    Xq, sx = quant(inp["X"], T, d)
    logits = torch.empty(T, E, **f32)
    act = None if mx else torch.empty(R_max, n, dtype=torch.bfloat16, device="cuda")
    act_q = torch.empty(R_max, n, **u8)
    sact = torch.empty(B.moe_mx_scale_bytes(R_max, n), **u8) if mx else torch.empty(R_max, **f32)
    Y = torch.empty(R_max, d, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    ws_r, nb_r = B.workspace(dims, B.OP_ROUTE)
    ws_q, nb_q = B.workspace(dims, B.OP_FFN_MX if mx else B.OP_FFN_FP8)
    ws_f, nb_f = B.workspace(dims, B.OP_FORWARD)
    out_bf = torch.empty_like(out)

    def step():
        B.moe_route(dims, inp["X"], inp["W_r"], inp["bias"], logits, plan, ws_r, nb_r)
        if mx:
            B.moe_quantize_mx(inp["X"], fmt, Xq, sx)
            B.moe_grouped_ffn_mx(dims, plan, fmt, Xq, sx, Wgq, sg, Wuq, su, Wdq, sd, None, act_q, sact, Y, ws_q, nb_q)
        else:
            B.moe_quantize_fp8(inp["X"], Xq, sx)
            B.moe_grouped_ffn_fp8(dims, plan, Xq, sx, Wgq, sg, Wuq, su, Wdq, sd, act, act_q, sact, Y, ws_q, nb_q)
        B.moe_combine(dims, plan, Y, 1, out)

    def bf16_step():
        B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                      logits, plan, None, out_bf, ws_f, nb_f)

    def timed(fn, with_stages):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        if with_stages:
            B.moe_timing_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        st = {s: B.moe_timing_read(s) for s in B.STAGES} if with_stages else None
        if with_stages:
            B.moe_timing_enable(False)
        return e0.elapsed_time(e1) / args.steps, st

    ms_bf, _ = timed(bf16_step, False)
    ms, stages = timed(step, True)
    R = int(plan.meta[0].item())
    rel = float((out.float() - out_bf.float()).abs().max() / out_bf.float().abs().max())
    flops = 6 * R * d * n + 2 * T * d * E
    value = flops / (ms * 1e-3) / 1e12
    stage_fl = {"router_gemm": 2 * T * d * E, "fp8_up_gemm": 4 * R * d * n, "fp8_down_gemm": 2 * R * d * n}
    breakdown = {}
    for s_, v in stages.items():
        if not v:
            continue
        avg = float(np.mean(v))
        ent = {"launches_per_step": round(len(v) / args.steps, 3), "avg_ms": round(avg, 4),
               "ms_per_step": round(float(np.sum(v)) / args.steps, 4)}
        if s_ in stage_fl:
            ent["tflops"] = round(stage_fl[s_] / (avg * 1e-3) / 1e12, 1)
        breakdown[s_] = ent
    dom = max(("fp8_up_gemm", "fp8_down_gemm"), key=lambda s_: breakdown[s_]["ms_per_step"])
    avg = breakdown[dom]["avg_ms"]
    ach = stage_fl[dom] / (avg * 1e-3) / 1e12
    scaling = ("%s, 32-element E8M0 block scales" % args.mx.upper()) if mx else "E4M3, per-row scales"
    res = {
        "metric": "MoE layer fwd useful TFLOPS, FP8 (%s) expert GEMMs, %s" % (scaling, cfg.name),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8_%s (block scales)" % args.mx) if mx else "fp8_e4m3 (bf16 activations between the GEMMs)",
        "data": "synthetic (seeded normal inputs and random-init weights)",
        "config": {"workload": cfg.name, "T": T, "d": d, "n": n, "E": E, "K": cfg.K, "pass": "fwd", "rows": R,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_FP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None, "avg_ms": avg},
        "bf16_forward_ms": round(ms_bf, 4),
        "speedup_vs_bf16_forward": round(ms_bf / ms, 3),
        "max_rel_diff_vs_bf16_forward": round(rel, 4),
        "stages": breakdown,
    }
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(requested --gpus %d, WORLD_SIZE=%d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)
    if args.decode:
        return decode_bench(args)
    if args.fp8 or args.mx:
        return fp8_bench(args)
    import torch
    from mixture_experts_layer_lds_amd import binding as B
    from mixture_experts_layer_lds_amd import workloads as wl

    cfg = wl.BY_NAME[args.config]
    if args.round_mode is not None:
        cfg = cfg.with_(round_mode=args.round_mode)
    if args.tile_m is not None:
        cfg = cfg.with_(tile_m=args.tile_m)
    backward = cfg.backward and not args.forward_only
    log("config", cfg)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=backward)
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype, cfg.round_mode, cfg.tile_m,
                       inp["round_rand"])
    dt = B.torch_dtype(dims)
    plan = B.Plan(dims)
    R_max = plan.R_max
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    H = torch.empty(R_max, 2 * cfg.n, dtype=dt, device="cuda") if backward else None
    out = torch.empty(cfg.T, cfg.d, dtype=dt, device="cuda")
    ws_f, nb_f = B.workspace(dims, B.OP_FORWARD)
    if backward:
        g = dict(dX=torch.empty_like(inp["X"]), dW_gate=torch.empty_like(inp["W_gate"]),
                 dW_up=torch.empty_like(inp["W_up"]), dW_down=torch.empty_like(inp["W_down"]),
                 dS=torch.empty(R_max, dtype=torch.float32, device="cuda"),
                 dLogits=torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda"),
                 dW_r=torch.empty_like(inp["W_r"]))
        ws_b, nb_b = B.workspace(dims, B.OP_BACKWARD)
    h_arg = None if args.no_h_cache else H

    def step():
        B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                      logits, plan, H, out, ws_f, nb_f)
        if backward:
            B.moe_backward(dims, inp["dY"], inp["X"], inp["W_r"], inp["W_gate"], inp["W_up"], inp["W_down"],
                           plan, h_arg, g["dX"], g["dW_gate"], g["dW_up"], g["dW_down"], g["dS"],
                           g["dLogits"], g["dW_r"], ws_b, nb_b)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    R = int(plan.meta[0].item())
    log("warmup done, R =", R)
    if args.calibrate_copy:
        src = torch.ones(1 << 26, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
        log("calibration copy: 3 x (256 MiB read + 256 MiB written)")

    # headline: K steps with the library's stage timing off; one event per step boundary gives the
    # per-step distribution
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    total_ms = evs[0].elapsed_time(evs[-1])
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_step = total_ms / args.steps
    log("timed %d steps: %.3f ms/step (median %.3f, min %.3f)"
        % (args.steps, ms_step, float(np.median(per_step)), min(per_step)))

    # stage pass: the same K steps again with a hipEvent pair around every stage, recorded by the
    # library on the stream it launches on
    B.moe_timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    stage_pass_ms = e0.elapsed_time(e1) / args.steps
    stages = {s: B.moe_timing_read(s) for s in B.STAGES}
    B.moe_timing_enable(False)
    log("stage pass: %.3f ms/step" % stage_pass_ms)

    # the HBM-bound gather kernels on their own, each rep after a 1 GiB write that flushes the
    # 256 MB MALL and the L2s (inputs would otherwise stay cached between reps): combine of the
    # expert outputs, and the packed-mode permute, which the step does not run (its GEMMs gather
    # rows themselves) but which is the materialised dispatch of the same plan
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    Y_perm = torch.empty(R_max, cfg.d, dtype=dt, device="cuda")
    H_tmp = torch.empty(R_max, 2 * cfg.n, dtype=dt, device="cuda")
    ws_ffn, nb_ffn = B.workspace(dims, B.OP_FFN)
    B.moe_grouped_ffn(dims, plan, inp["X"], 1, inp["W_gate"], inp["W_up"], inp["W_down"], H_tmp, Y_perm,
                      ws_ffn, nb_ffn)
    del H_tmp, ws_ffn
    X_perm = torch.empty(R_max, cfg.d, dtype=dt, device="cuda")
    out_c = torch.empty_like(out)
    B.moe_timing_enable(True)
    for i in range(args.steps):
        flush.fill_(i & 255)
        B.moe_combine(dims, plan, Y_perm, 1, out_c)
        flush.fill_((i + 7) & 255)
        B.moe_permute(dims, plan, inp["X"], X_perm)
    torch.cuda.synchronize()
    flushed = {"combine": B.moe_timing_read("combine"), "permute": B.moe_timing_read("permute")}
    B.moe_timing_enable(False)
    # the practical ceiling of the same protocol: torch's device copy of the combine's byte count
    # (half read, half written), each rep after the same flush
    nb_copy = stage_bytes("combine", R, cfg.T, cfg.d, cfg.n, cfg.E, 2 if cfg.dtype == "bf16" else 4, cfg.K) // 2
    csrc = torch.ones(nb_copy // 16, 4, dtype=torch.float32, device="cuda")
    cdst = torch.empty_like(csrc)
    copy_ms = []
    for i in range(args.steps):
        flush.fill_(i & 255)
        e0.record()
        cdst.copy_(csrc)
        e1.record()
        torch.cuda.synchronize()
        copy_ms.append(e0.elapsed_time(e1))
    del flush, Y_perm, X_perm, out_c, csrc, cdst

    # the backward recomputing [G|U] from X instead of reading the forward's H cache
    recompute_ms = None
    if backward and not args.no_h_cache:
        def step_recompute():
            B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                          logits, plan, None, out, ws_f, nb_f)
            B.moe_backward(dims, inp["dY"], inp["X"], inp["W_r"], inp["W_gate"], inp["W_up"], inp["W_down"],
                           plan, None, g["dX"], g["dW_gate"], g["dW_up"], g["dW_down"], g["dS"],
                           g["dLogits"], g["dW_r"], ws_b, nb_b)
        for _ in range(args.warmup):
            step_recompute()
        e0.record()
        for i in range(args.steps):
            step_recompute()
        e1.record()
        torch.cuda.synchronize()
        recompute_ms = e0.elapsed_time(e1) / args.steps
        log("recompute step: %.3f ms" % recompute_ms)

    T, d, n, E = cfg.T, cfg.d, cfg.n, cfg.E
    es = 2 if cfg.dtype == "bf16" else 4
    flops = 6 * R * d * n + 2 * T * d * E
    if backward:
        flops += 12 * R * d * n + 4 * T * d * E
    value = flops / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS

    # the counter record is per exact workload: shape, pass, token rounding and H cache
    workload_key = "%s:%s:round%d%s:%s" % (cfg.name, "fwd+bwd" if backward else "fwd", cfg.round_mode,
                                           (":tile%d" % cfg.tile_m) if cfg.round_mode else "",
                                           ("h_cache" if not args.no_h_cache else "recompute") if backward else "-")
    breakdown = {}
    for s, v in stages.items():
        if not v:
            continue
        avg = float(np.mean(v))
        ent = {"launches_per_step": round(len(v) / args.steps, 3), "avg_ms": round(avg, 4),
               "median_ms": round(float(np.median(v)), 4), "min_ms": round(float(np.min(v)), 4),
               "ms_per_step": round(float(np.sum(v)) / args.steps, 4)}
        f = stage_flops(s, R, T, d, n, E)
        b = stage_bytes(s, R, T, d, n, E, es, cfg.K)
        if f:
            ent["tflops"] = round(f / (avg * 1e-3) / 1e12, 1)
            ent["pct_peak"] = round(100 * f / (avg * 1e-3) / 1e12 / peak, 1)
        if b:
            ent["gbs"] = round(b / (avg * 1e-3) / 1e9, 1)
            ent["pct_hbm"] = round(100 * b / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 1)
        breakdown[s] = ent
    gemm_stages = [s for s in breakdown if stage_flops(s, R, T, d, n, E)]
    modelled = [s for s in breakdown if
                (stage_flops(s, R, T, d, n, E) or stage_bytes(s, R, T, d, n, E, es, cfg.K))]
    hbm_flushed = {}
    for s, v in flushed.items():
        b = stage_bytes(s, R, T, d, n, E, es, cfg.K)
        med, mn = float(np.median(v)), float(np.min(v))
        hbm_flushed[s] = {"reps": len(v), "median_ms": round(med, 4), "min_ms": round(mn, 4),
                          "bytes": int(b), "gbs_median": round(b / (med * 1e-3) / 1e9, 1),
                          "gbs_best": round(b / (mn * 1e-3) / 1e9, 1),
                          "pct_hbm_median": round(100 * b / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 1),
                          "in_step": s != "permute"}
    cb = 2 * (stage_bytes("combine", R, T, d, n, E, es, cfg.K) // 2 // 16) * 16
    hbm_flushed["copy_reference"] = {"reps": len(copy_ms), "median_ms": round(float(np.median(copy_ms)), 4),
                                     "bytes": int(cb),
                                     "gbs_median": round(cb / (float(np.median(copy_ms)) * 1e-3) / 1e9, 1),
                                     "pct_hbm_median": round(100 * cb / (float(np.median(copy_ms)) * 1e-3) / 1e9
                                                             / PEAK_HBM_GBS, 1),
                                     "what": "torch device copy of the combine's byte count, half read and half written"}
    dom = max(modelled, key=lambda s: breakdown[s]["ms_per_step"])
    if stage_flops(dom, R, T, d, n, E):
        avg = breakdown[dom]["avg_ms"]
        ach = stage_flops(dom, R, T, d, n, E) / (avg * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": measured_traffic(workload_key, dom), "avg_ms": avg,
                "algorithmic_bytes": stage_min_bytes(dom, R, T, d, n, E, es)}
    else:
        avg = breakdown[dom]["avg_ms"]
        ach = stage_bytes(dom, R, T, d, n, E, es, cfg.K) / (avg * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": measured_traffic(workload_key, dom), "avg_ms": avg,
                "algorithmic_bytes": stage_bytes(dom, R, T, d, n, E, es, cfg.K)}
    gemm_ms = sum(breakdown[s]["ms_per_step"] for s in gemm_stages)
    expert_flops = (18 if backward else 6) * R * d * n
    res = {
        "metric": METRIC if (cfg.name == "fine_grained_7b" and backward) else
        "MoE layer %s useful TFLOPS, %s" % ("fwd+bwd" if backward else "fwd", cfg.name),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded normal inputs and random-init weights)",
        "config": {"workload": cfg.name, "key": workload_key, "T": T, "d": d, "n": n, "E": E, "K": cfg.K,
                   "pass": "fwd+bwd" if backward else "fwd", "round_mode": cfg.round_mode,
                   "tile_m": cfg.tile_m, "rows": R, "h_cache": (not args.no_h_cache) if backward else None,
                   "parallelism": "single GPU"},
        "pct_bf16_peak": round(100 * value / peak, 2),
        "grouped_gemm_pct_peak": round(100 * expert_flops / (gemm_ms * 1e-3) / 1e12 / peak, 2) if gemm_ms else None,
        "roofline": roof,
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_min": round(float(np.min(per_step)), 4),
        "stage_pass_ms_per_step": round(stage_pass_ms, 4),
        "stages": breakdown,
        "hbm_kernels_flushed": hbm_flushed,
        "memory": memory_accounting(cfg, dims, R_max, backward, B),
    }
    if recompute_ms is not None:
        res["no_h_cache"] = {"ms_per_step": round(recompute_ms, 4),
                             "value": round(flops / (recompute_ms * 1e-3) / 1e12, 2)}
    if not args.no_cpu:
        log("CPU oracle baseline ...")
        res["cpu_baseline"] = cpu_baseline(cfg, inp, logits, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

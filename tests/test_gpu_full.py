"""GPU parity at the full sizes of the five layer workloads, in the launch configuration the
benchmark times, and on two shapes chosen for launch paths that small cases do not reach.

* Fine-grained 7B-style layer (forward + backward) and Mixtral-shaped layer (forward): every output
  element by element against the float64 oracle run on the whole layer.  Routing is bit-exact over
  every row (the oracle rebuilds the plan from the GPU's fp32 logits); logits, out and H are
  compared in full and, with the backward, dX, dS, dLogits, dW_gate / dW_up / dW_down of every
  expert and dW_r, the latter against the oracle's own dLogits^T X.
* DeepSeek-V3- and Kimi-K2-shaped layers (a whole-layer float64 oracle takes minutes): routing
  bit-exact over every row; every row of three whole experts -- the most-loaded one (the longest
  weight-gradient reductions), the least-loaded non-empty one and the median one -- for H and
  Y_perm (Y_perm from moe_grouped_ffn on the same plan, the kernels moe_forward runs) and, with the
  backward, their dS rows and dW_gate / dW_up / dW_down; and sampled tokens (logits, out, dX, dS
  and dLogits through the plan restricted to those tokens, whose dS the oracle computes itself).
* A medium layer whose every GEMM launches more than 256 workgroups (several rounds of the grid
  and full XCD chunks of the tile remap), compared in full, forward and backward.
* T = 33000 tokens with token rounding: the rounding kernel's path for T > 32768, where an
  expert's keys do not fit in LDS; routing bit-exact, forward and backward in full.
"""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_lds_amd import workloads as wl
from conftest import announce_case, progress
from parity import (TOL, ExpertSubset, assert_close, check_backward, check_forward, check_routing,
                    compact_plan, run_gpu, run_grouped_ffn, subset_plan)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


class GpuExperts:
    """W[e] as float64 numpy, converted on the GPU one expert at a time and cached."""

    def __init__(self, t):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].to(torch.float64).cpu().numpy()
        return self.cache[e]

    def __len__(self):
        return self.t.shape[0]


def gpu_f64(t):
    return t.to(torch.float64).cpu().numpy()


def sample_tokens(T, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=k, replace=False))


def pick_experts(counts):
    """The most-loaded expert, the least-loaded non-empty one and the median one."""
    nz = np.nonzero(counts)[0]
    order = np.argsort(counts, kind="stable")
    return sorted({int(np.argmax(counts)), int(nz[np.argmin(counts[nz])]), int(order[len(order) // 2])})


def run_whole(cfg):
    """Every output of the layer against the oracle on the whole layer."""
    progress("GPU layer")
    res = run_gpu(cfg)
    ref = check_routing(cfg, res)                      # every row, bit-exact
    progress("routing bit-exact; oracle forward")
    errs, _ = check_forward(cfg, res, ref)
    if cfg.backward:
        progress("oracle backward")
        errs.update(check_backward(cfg, res, ref))
    progress("max relative errors: " + ", ".join("%s %.2e" % kv for kv in sorted(errs.items())))
    return res, ref


def run_sampled(cfg, n_tokens):
    """Routing in full; three whole experts and sampled tokens against the oracle."""
    progress("GPU layer")
    res = run_gpu(cfg)
    ref = check_routing(cfg, res)                      # every row, bit-exact
    inp = res["inputs"]
    tol = TOL[cfg.dtype]
    X = gpu_f64(inp["X"])
    Wg, Wu, Wd = GpuExperts(inp["W_gate"]), GpuExperts(inp["W_up"]), GpuExperts(inp["W_down"])
    errs = {}

    # sampled tokens: logits, out, the tokens' H rows and, with the backward, dX, dS, dLogits.  The
    # plan restricted to the tokens is renumbered to the experts they use, so the oracle touches
    # only those experts' weights.
    toks = sample_tokens(cfg.T, n_tokens, cfg.index)
    sub, rows = subset_plan(ref, toks)
    subc, used = compact_plan(sub)
    Wgs, Wus, Wds = ExpertSubset(Wg, used), ExpertSubset(Wu, used), ExpertSubset(Wd, used)
    tt = torch.from_numpy(toks).cuda()
    bias = None if inp["bias"] is None else gpu_f64(inp["bias"])
    W_r = gpu_f64(inp["W_r"])
    L_ref = oracle.router_logits(X[toks], W_r, bias)
    errs["logits"] = assert_close("logits", gpu_f64(res["logits"][tt]), L_ref, tol)
    progress("tokens %s on %d experts: oracle forward" % ([int(t) for t in toks], len(used)))
    fw = oracle.layer_forward(X, Wgs, Wus, Wds, subc)
    errs["out"] = assert_close("out", gpu_f64(res["out"][tt]), fw["out"][toks], tol)
    rows_t = torch.from_numpy(rows).cuda()
    errs["H(tokens)"] = assert_close("H", gpu_f64(res["H"][rows_t]), fw["H"], tol)
    if cfg.backward:
        progress("tokens: oracle backward")
        dY = gpu_f64(inp["dY"])
        bw = oracle.layer_backward(dY, X, Wgs, Wus, Wds, subc, W_r=W_r[used])
        dL = np.zeros((cfg.T, cfg.E))
        dL[:, used] = bw["dLogits"]
        errs["dX"] = assert_close("dX", gpu_f64(res["dX"][tt]), bw["dX"][toks], tol)
        errs["dS(tokens)"] = assert_close("dS", gpu_f64(res["dS"][rows_t]), bw["dS"], tol)
        errs["dLogits"] = assert_close("dLogits", gpu_f64(res["dLogits"][tt]), dL[toks], tol)

    # whole experts: every row of H and Y_perm, their dS rows and their weight gradients
    picks = pick_experts(ref["counts"])
    _, Y = run_grouped_ffn(cfg, res)
    off = ref["expert_off"]
    progress("experts %s with %s rows: oracle forward" % (picks, [int(ref["counts"][e]) for e in picks]))
    fwe = oracle.layer_forward(X, Wg, Wu, Wd, ref, experts=picks)
    if cfg.backward:
        progress("experts: oracle backward")
        bwe = oracle.layer_backward(gpu_f64(inp["dY"]), X, Wg, Wu, Wd, ref, experts=picks)
    for e in picks:
        lo, hi = int(off[e]), int(off[e + 1])
        errs["H[%d]" % e] = assert_close("H[%d]" % e, gpu_f64(res["H"][lo:hi]), fwe["H"][lo:hi], tol)
        errs["Y_perm[%d]" % e] = assert_close("Y_perm[%d]" % e, gpu_f64(Y[lo:hi]), fwe["Y_perm"][lo:hi], tol)
        if cfg.backward:
            errs["dS[%d]" % e] = assert_close("dS[%d]" % e, gpu_f64(res["dS"][lo:hi]), bwe["dS"][lo:hi], tol)
            for k in ("dW_gate", "dW_up", "dW_down"):
                errs["%s[%d]" % (k, e)] = assert_close("%s[%d]" % (k, e), gpu_f64(res[k][e]), bwe[k][e], tol)
    progress("max relative errors: " + ", ".join("%s %.2e" % kv for kv in sorted(errs.items())))
    return res, ref, picks


def test_full_fine_grained_forward_backward():
    """The benchmark's layer (T=32768, d=1536, E=128, K=8, n=256), every output in full."""
    run_whole(wl.BY_NAME["fine_grained_7b"])


def test_full_mixtral_coarse_forward():
    """T=8192, d=4096, E=8, K=2, n=14336: every output in full."""
    cfg = wl.BY_NAME["mixtral_coarse"]
    res, ref = run_whole(cfg)
    c = ref["counts"]
    assert c.sum() == cfg.T * cfg.K and c.min() > 0.8 * c.mean()      # near-uniform routing


def test_full_deepseek_v3_forward():
    cfg = wl.BY_NAME["deepseek_v3"]
    res, ref, picks = run_sampled(cfg, n_tokens=6)
    c = ref["counts"]
    assert c.max() > 2 * c[c > 0].min()                                # the bias skews the loads


@pytest.mark.parametrize("mode", [0, 1])
def test_full_kimi_k2_forward_backward(mode):
    cfg = wl.BY_NAME["kimi_k2"].with_(round_mode=mode, tile_m=128)
    res, ref, picks = run_sampled(cfg, n_tokens=4)
    if mode:
        assert np.all(ref["counts"] % 128 == 0)
    assert max(ref["counts"]) > 4 * 256                                # the hot expert spans many M-tiles


def test_medium_layer_with_multi_round_grids():
    """T=8000, d=1536, E=32, K=4, n=768, bias N(0,1): R = 32000 rows, so every expert GEMM has more
    tiles than 256 CUs hold at once (at the mean load of 1000 rows: gate/up 768, down 1536, dAct
    384, dX 768, dW_down 576, dW_gate/up 1152), and the grids run several rounds through the XCD
    tile remap.  Forward and backward compared in full."""
    cfg = wl.small_shape(T=8000, d=1536, E=32, K=4, n=768, dtype="bf16", bias="normal", seed=71)
    res, ref = run_whole(cfg)
    assert ref["counts"].max() > 2 * 256


@pytest.mark.parametrize("mode", [1, 4])
def test_token_rounding_above_lds_cached_tokens(mode):
    """T = 33000 > 32768: the rounding kernel ranks an expert's tokens straight from global memory
    instead of an LDS copy.  Nearest and stochastic rounding to 128, routing bit-exact, forward and
    backward in full."""
    cfg = wl.small_shape(T=33000, d=128, E=8, K=2, n=128, dtype="bf16", round_mode=mode, tile_m=128,
                         seed=73)
    res, ref = run_whole(cfg)
    assert np.all(ref["counts"] % 128 == 0)
    assert not np.array_equal(ref["counts"], np.bincount(ref["topk_idx"].ravel(), minlength=cfg.E))

"""GPU parity at the full sizes of the five layer workloads, in the launch configuration the
benchmark times.  Routing is checked bit-exactly over every row (the oracle rebuilds the plan from
the GPU's fp32 logits); floating-point outputs are checked on outputs the oracle can compute one
by one: sampled tokens (their output, dX, dS, dLogits and logits rows, through the plan
restricted to those tokens) and sampled experts (their weight gradients); the router weight
gradient is checked through its defining identity dW_r = dLogits^T X at full size.
"""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_lds_amd import workloads as wl
from conftest import announce_case
from parity import (TOL, assert_close, check_routing, f64, run_gpu, subset_plan)

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


def gpu_f64(t):
    return t.to(torch.float64).cpu().numpy()


def sample_tokens(T, k, seed):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, size=k, replace=False))


def run_full(cfg, n_tokens=6, backward=None):
    res = run_gpu(cfg, backward=backward)
    ref = check_routing(cfg, res)                      # every row, bit-exact
    inp = res["inputs"]
    tol = TOL[cfg.dtype]
    toks = sample_tokens(cfg.T, n_tokens, cfg.index)
    sub, rows = subset_plan(ref, toks)
    X = gpu_f64(inp["X"])
    bias = None if inp["bias"] is None else gpu_f64(inp["bias"])
    L_ref = oracle.router_logits(X[toks], gpu_f64(inp["W_r"]), bias)
    assert_close("logits", gpu_f64(res["logits"][torch.from_numpy(toks).cuda()]), L_ref, tol)
    Wg, Wu, Wd = GpuExperts(inp["W_gate"]), GpuExperts(inp["W_up"]), GpuExperts(inp["W_down"])
    fw = oracle.layer_forward(X, Wg, Wu, Wd, sub)
    assert_close("out", gpu_f64(res["out"][torch.from_numpy(toks).cuda()]), fw["out"][toks], tol)
    rows_t = torch.from_numpy(rows).cuda()
    assert_close("H", gpu_f64(res["H"][rows_t]), fw["H"], tol)
    if backward if backward is not None else cfg.backward:
        dY = gpu_f64(inp["dY"])
        bw = oracle.layer_backward(dY, X, Wg, Wu, Wd, sub, W_r=gpu_f64(inp["W_r"]))
        tt = torch.from_numpy(toks).cuda()
        assert_close("dX", gpu_f64(res["dX"][tt]), bw["dX"][toks], tol)
        assert_close("dS", gpu_f64(res["dS"][rows_t]), bw["dS"], tol)
        assert_close("dLogits", gpu_f64(res["dLogits"][tt]), bw["dLogits"][toks], tol)
        # sampled experts: the least-loaded non-empty expert and the median-loaded one
        counts = ref["counts"]
        nz = np.nonzero(counts)[0]
        picks = sorted({int(nz[np.argmin(counts[nz])]), int(np.argsort(counts)[len(counts) // 2])})
        bwe = oracle.layer_backward(dY, X, Wg, Wu, Wd, ref, experts=picks)
        for e in picks:
            assert_close("dW_gate[%d]" % e, gpu_f64(res["dW_gate"][e]), bwe["dW_gate"][e], tol)
            assert_close("dW_up[%d]" % e, gpu_f64(res["dW_up"][e]), bwe["dW_up"][e], tol)
            assert_close("dW_down[%d]" % e, gpu_f64(res["dW_down"][e]), bwe["dW_down"][e], tol)
        # router weight gradient: its definition applied to the GPU's (sample-checked) dLogits
        dWr_def = gpu_f64(res["dLogits"]).T @ X
        assert_close("dW_r", gpu_f64(res["dW_r"]), dWr_def, tol)
    return res, ref


def test_full_mixtral_coarse_forward():
    cfg = wl.BY_NAME["mixtral_coarse"]
    res, ref = run_full(cfg)
    c = ref["counts"]
    assert c.sum() == cfg.T * cfg.K and c.min() > 0.8 * c.mean()      # near-uniform routing


def test_full_fine_grained_forward_backward():
    run_full(wl.BY_NAME["fine_grained_7b"])


def test_full_deepseek_v3_forward():
    run_full(wl.BY_NAME["deepseek_v3"])


@pytest.mark.parametrize("mode", [0, 1])
def test_full_kimi_k2_forward_backward(mode):
    cfg = wl.BY_NAME["kimi_k2"].with_(round_mode=mode, tile_m=128)
    res, ref = run_full(cfg, n_tokens=4)
    if mode:
        assert np.all(ref["counts"] % 128 == 0)

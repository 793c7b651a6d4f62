"""GPU parity of the single-launch decode path (moe_decode) against the float64 oracle.

The decode call must compute the same layer as moe_forward with plain top-K: routing bit-exact
given its own fp32 logits (which must match the oracle's X W_r^T + b within the layer's
tolerance), outputs within max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2 bf16).
"""
import numpy as np
import pytest
import torch

import oracle
from conftest import announce_case
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl
from parity import TOL, assert_close, f64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


class GpuExperts:
    """W[e] as float64 numpy, converted one expert at a time (only the experts a check uses)."""

    def __init__(self, t):
        self.t = t
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self.t[e].to(torch.float64).cpu().numpy()
        return self.cache[e]


def run_decode(cfg, inp):
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype)
    dt = B.torch_dtype(dims)
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    topk_idx = torch.empty(cfg.T, cfg.K, dtype=torch.int32, device="cuda")
    topk_w = torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda")
    out = torch.empty(cfg.T, cfg.d, dtype=dt, device="cuda")
    ws, nb = B.workspace(dims, B.OP_DECODE)
    B.moe_decode(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                 logits, topk_idx, topk_w, out, ws, nb)
    torch.cuda.synchronize()
    return logits, topk_idx, topk_w, out


def check_decode(cfg, inp, logits, topk_idx, topk_w, out):
    tol = TOL[cfg.dtype]
    X = f64(inp["X"])
    bias = f64(inp["bias"]) if inp["bias"] is not None else None
    assert_close("logits", f64(logits), oracle.router_logits(X, f64(inp["W_r"]), bias), tol)
    L = f64(logits)
    ref = oracle.build_plan(L, cfg.K)
    assert np.array_equal(topk_idx.cpu().numpy(), ref["topk_idx"]), "topk_idx"
    assert_close("topk_w", f64(topk_w), ref["topk_w"], tol)
    want = oracle.token_forward(X, GpuExperts(inp["W_gate"]), GpuExperts(inp["W_up"]),
                                GpuExperts(inp["W_down"]), ref, np.arange(cfg.T))
    return assert_close("out", f64(out), want, tol)


@pytest.mark.parametrize("T,dtype", [(1, "bf16"), (3, "f32"), (17, "bf16"), (64, "bf16"), (40, "f32"),
                                     (200, "bf16"), (130, "f32")])
def test_decode_small_shapes(T, dtype):
    """T = 200 and 130 give experts with 33 to 64 tokens: passes of three token groups and a
    partial last pass."""
    cfg = wl.small_shape(T=T, d=256, E=16, K=4, n=192, dtype=dtype, bias="normal", backward=False,
                         seed=60 + T)
    inp = wl.make_inputs(cfg, device="cuda")
    print(check_decode(cfg, inp, *run_decode(cfg, inp)))


def test_decode_single_expert_and_all_experts():
    for E, K in ((1, 1), (6, 6)):
        cfg = wl.small_shape(T=9, d=128, E=E, K=K, n=64, dtype="f32", backward=False, seed=70 + E)
        inp = wl.make_inputs(cfg, device="cuda")
        check_decode(cfg, inp, *run_decode(cfg, inp))


def test_decode_matches_forward():
    """Same layer as moe_forward (plain top-K) up to the fp32-vs-dtype activation rounding."""
    cfg = wl.small_shape(T=32, d=512, E=32, K=8, n=256, dtype="bf16", backward=False, seed=81)
    inp = wl.make_inputs(cfg, device="cuda")
    logits, topk_idx, topk_w, out = run_decode(cfg, inp)
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16")
    plan = B.Plan(dims)
    lf = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    of = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
    ws, nb = B.workspace(dims, B.OP_FORWARD)
    B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                  lf, plan, None, of, ws, nb)
    torch.cuda.synchronize()
    assert_close("logits vs forward", f64(logits), f64(lf), TOL["bf16"])
    assert_close("out vs forward", f64(out), f64(of), TOL["bf16"])


@pytest.mark.slow
@pytest.mark.parametrize("name,T", [("deepseek_v3", 4), ("fine_grained_7b", 16), ("kimi_k2", 2)])
def test_decode_full_layer_shapes(name, T):
    base = wl.BY_NAME[name]
    cfg = base.with_(T=T, backward=False, round_mode=0)
    inp = wl.make_inputs(cfg, device="cuda")
    print(check_decode(cfg, inp, *run_decode(cfg, inp)))


def test_decode_calls_on_two_streams_do_not_overlap():
    """Decode calls on different streams (each with its own workspace) give the same bits as the
    same calls on one stream: each call's grid barriers count in its own workspace, so calls share
    no device state, and no call reports a barrier that gave up."""
    cfgs = [wl.small_shape(T=24, d=512, E=32, K=4, n=256, dtype="bf16", backward=False, seed=s)
            for s in (91, 92)]
    inps = [wl.make_inputs(c, device="cuda") for c in cfgs]
    refs = [run_decode(c, i) for c, i in zip(cfgs, inps)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for rep in range(3):
        for j in (0, 1):
            cfg, inp = cfgs[j], inps[j]
            dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype)
            with torch.cuda.stream(streams[j]):
                o = [torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda"),
                     torch.empty(cfg.T, cfg.K, dtype=torch.int32, device="cuda"),
                     torch.empty(cfg.T, cfg.K, dtype=torch.float32, device="cuda"),
                     torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")]
                ws, nb = B.workspace(dims, B.OP_DECODE)
                B.moe_decode(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"],
                             inp["W_down"], *o, ws, nb, stream=streams[j])
                outs.append((j, o, ws))
    torch.cuda.synchronize()
    B.moe_decode_status()
    for j, o, _ in outs:
        for got, want in zip(o, refs[j]):
            assert torch.equal(got, want)


def test_decode_barrier_give_up_is_reported():
    """The give-up path of the grid barrier, forced from the host: with a spin limit of 0 every
    workgroup gives up at the first barrier without polling (it never waits, so every workgroup
    leaves the kernel normally).  moe_decode_status then raises MOE_EHIP once and clears the status
    word; the next call with the default limit matches a clean call bit for bit and reports
    nothing."""
    cfg = wl.small_shape(T=16, d=256, E=16, K=2, n=128, dtype="bf16", backward=False, seed=93)
    inp = wl.make_inputs(cfg, device="cuda")
    ref = run_decode(cfg, inp)
    B.moe_decode_status()                                  # nothing pending
    prev = B.moe_decode_set_spin_limit(0)
    try:
        run_decode(cfg, inp)
    finally:
        assert B.moe_decode_set_spin_limit(prev) == 0
    with pytest.raises(B.MoEError) as err:
        B.moe_decode_status()
    assert err.value.status == -4 and "grid barrier" in str(err.value)
    B.moe_decode_status()                                  # cleared by the read
    again = run_decode(cfg, inp)
    B.moe_decode_status()
    for got, want in zip(again, ref):
        assert torch.equal(got, want)

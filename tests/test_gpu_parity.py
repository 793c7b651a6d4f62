"""GPU parity: the HIP library (through its C ABI) against the float64 oracle, element by element,
on seeded inputs small enough for the oracle but spanning several GEMM tiles with ragged tails.

Routing outputs must be bit-exact given the same fp32 logits; floating-point outputs and
gradients must satisfy max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2 bf16).
"""

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl
from conftest import announce_case
from parity import (TOL, assert_close, check_backward, check_forward, check_routing, f64, run_gpu)

pytestmark = pytest.mark.gpu



@pytest.fixture(autouse=True)
def announce(request):
    """Record which case is about to touch the GPU, flushed before it runs."""
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield


def full_check(cfg, **kw):
    res = run_gpu(cfg, **kw)
    ref = check_routing(cfg, res)
    errs, _ = check_forward(cfg, res, ref)
    if cfg.backward:
        errs.update(check_backward(cfg, res, ref))
    return res, ref, errs


def test_tiny_fp32_layer_forward_backward():
    cfg = wl.BY_NAME["tiny_fp32"].with_(backward=True)
    _, ref, errs = full_check(cfg)
    assert int(ref["counts"].sum()) == cfg.T * cfg.K
    print(errs)


@pytest.mark.parametrize("shape", [
    dict(T=1000, d=192, E=4, K=2, n=320, dtype="bf16"),
    dict(T=700, d=128, E=5, K=3, n=192, dtype="f32"),
    dict(T=333, d=256, E=16, K=4, n=128, dtype="bf16"),
    dict(T=129, d=64, E=3, K=1, n=64, dtype="f32"),
    dict(T=400, d=192, E=3, K=2, n=576, dtype="bf16"),  # n > 512: the four-wave bf16 down GEMM
    dict(T=1500, d=320, E=6, K=2, n=256, dtype="bf16"),  # down GEMM with LDS-held rows: 2 n-tiles, the last 64 wide
    dict(T=250, d=64, E=3, K=2, n=128, dtype="bf16"),    # the same with n = 128: one n-tile, 64 columns of 256
])
def test_ragged_multi_tile(shape):
    cfg = wl.small_shape(**shape, seed=31)
    _, _, errs = full_check(cfg)
    print(errs)


@pytest.mark.parametrize("shape", [
    dict(T=300, d=512, E=200, K=4, n=128),  # 2 x 2 ragged router tiles: d summed in 4 slices
    dict(T=520, d=192, E=136, K=2, n=64),   # 3 x 2 tiles: 2 slices of 3 k-steps each
])
def test_split_router_with_bias(shape):
    """bf16 layers whose router GEMM has few tiles split its reduction over d; the slices are
    added by top-K, which writes the final logits.  With a per-expert bias (added once, in the
    first slice), ragged token and expert tiles, and top-K over 16-lane rows (E <= 256)."""
    cfg = wl.small_shape(**shape, dtype="bf16", bias="normal", seed=37)
    _, _, errs = full_check(cfg)
    print(errs)


@pytest.mark.parametrize("mode,tile_m,dtype", [
    (1, 128, "f32"), (1, 32, "bf16"), (2, 16, "bf16"), (3, 64, "f32"), (2, 128, "f32"), (3, 8, "bf16"),
    (4, 128, "bf16"), (4, 16, "f32"),
])
def test_token_rounding_layer(mode, tile_m, dtype):
    cfg = wl.small_shape(T=900, d=128, E=6, K=2, n=128, dtype=dtype, bias="zipf", round_mode=mode,
                         tile_m=tile_m, seed=40 + mode)
    _, ref, errs = full_check(cfg)
    assert np.all(ref["counts"] % tile_m == 0)
    print(errs)


def test_single_expert_and_all_experts():
    full_check(wl.small_shape(T=200, d=128, E=1, K=1, n=128, dtype="f32", seed=5))
    full_check(wl.small_shape(T=200, d=128, E=4, K=4, n=64, dtype="f32", seed=6))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_limits_of_the_abi(dtype):
    """The largest expert count and top-K the library accepts (E = 1024, K = 16: sixteen
    candidates per lane in top-K, a 48 KiB router-backward row cache), a single token, and the
    smallest width (d = n = 64), forward and backward against the oracle."""
    _, ref, errs = full_check(wl.small_shape(T=300, d=64, E=1024, K=16, n=64, dtype=dtype, seed=11))
    assert int(ref["counts"].sum()) == 300 * 16
    print(errs)
    _, ref, errs = full_check(wl.small_shape(T=1, d=64, E=8, K=2, n=64, dtype=dtype, seed=12))
    assert int(ref["counts"].sum()) == 2
    print(errs)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_empty_experts(dtype):
    cfg = wl.small_shape(T=400, d=128, E=8, K=2, n=128, dtype=dtype, bias="normal", seed=7)
    inp = wl.make_inputs(cfg, device="cuda")
    inp["bias"] = torch.tensor([0, -100, 0, -100, 0, 0, -100, 0], dtype=torch.float32, device="cuda")
    res = run_gpu(cfg, inputs=inp)
    ref = check_routing(cfg, res)
    assert (ref["counts"] == 0).sum() == 3
    check_forward(cfg, res, ref)
    check_backward(cfg, res, ref)
    for e in (1, 3, 6):
        assert torch.count_nonzero(res["dW_gate"][e]) == 0
        assert torch.count_nonzero(res["dW_down"][e]) == 0


def test_recompute_equals_cached_and_determinism():
    cfg = wl.small_shape(T=512, d=256, E=8, K=2, n=192, dtype="bf16", seed=9)
    inp = wl.make_inputs(cfg, device="cuda")
    a = run_gpu(cfg, inputs=inp, cache_h=True)
    b = run_gpu(cfg, inputs=inp, cache_h=False)
    c = run_gpu(cfg, inputs=inp, cache_h=True)
    for k in ("out", "logits", "dX", "dW_gate", "dW_up", "dW_down", "dLogits", "dW_r"):
        assert torch.equal(a[k], b[k]), k
        assert torch.equal(a[k], c[k]), k
    R = int(a["plan"].meta[0])
    assert torch.equal(a["dS"][:R], b["dS"][:R])


@pytest.mark.parametrize("mode", [0, 1, 2, 3, 4])
def test_route_from_given_logits_with_ties(mode):
    """Caller-supplied logits with many exact ties (and -0.0): selection and indices bit-exact."""
    T, E, K = 777, 40, 5
    g = torch.Generator().manual_seed(123 + mode)
    L = torch.randint(-3, 4, (T, E), generator=g).to(torch.float32)
    L[::7] = 0.0
    L[3::11, ::2] = -0.0
    cfg = wl.small_shape(T=T, d=64, E=E, K=K, n=64, dtype="f32", round_mode=mode, tile_m=16)
    rr = wl.make_round_rand(cfg, "cuda")
    dims = B.make_dims(T, 64, 64, E, K, "f32", mode, 16, rr)
    plan = B.Plan(dims)
    logits = L.cuda()
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, None, None, None, logits, plan, ws, nb)
    torch.cuda.synchronize()
    check_routing(cfg, dict(plan=plan), L=L.double().numpy(), round_rand=rr)


@pytest.mark.parametrize("E,K", [(12, 3), (24, 4), (40, 8), (100, 8), (200, 16), (300, 8), (600, 16)])
def test_route_ties_and_nonfinite_in_every_selection_layout(E, K):
    """Top-K keeps four tokens per wave with 1, 2, 4, 8 or 16 keys per lane up to 256 experts and a
    wave per token above: exact ties, -0.0, NaN and infinities in every layout, plain top-K,
    selection, weights' order and the plan bit-exact against the oracle."""
    T = 333
    g = torch.Generator().manual_seed(1000 + E)
    L = torch.randint(-2, 3, (T, E), generator=g).to(torch.float32)
    L[::5] = 0.0
    L[1::9, ::3] = -0.0
    L[torch.rand(T, E, generator=g) < 0.1] = float("nan")
    L[torch.rand(T, E, generator=g) < 0.03] = float("inf")
    L[torch.rand(T, E, generator=g) < 0.03] = float("-inf")
    L[7, :] = float("nan")
    dims = B.make_dims(T, 64, 64, E, K, "f32")
    plan = B.Plan(dims)
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, None, None, None, L.cuda(), plan, ws, nb)
    torch.cuda.synchronize()
    got = plan.to_host()
    with np.errstate(invalid="ignore"):  # the softmax of a token with infinite logits
        ref = oracle.build_plan(L.double().numpy(), K)
    assert np.array_equal(got["topk_idx"].reshape(T, K), ref["topk_idx"])
    for k in ("counts", "expert_off", "row_token", "tok_off", "tok_row"):
        assert np.array_equal(got[k], ref[k]), k
    assert all(len(set(r.tolist())) == K for r in got["topk_idx"].reshape(T, K))


@pytest.mark.parametrize("round_mode", [2, 3])
def test_permute_after_token_rounding(round_mode):
    """Packed permute with token rounding: tokens with more than K rows (UP) or none (DOWN);
    every row r < R is a bit-exact copy of X[row_token[r]] and rows >= R are left untouched."""
    cfg = wl.small_shape(T=777, d=256, E=7, K=2, n=128, dtype="bf16", seed=29, round_mode=round_mode, tile_m=64)
    inp = wl.make_inputs(cfg, device="cuda")
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16", cfg.round_mode, cfg.tile_m)
    plan = B.Plan(dims)
    logits = torch.empty(cfg.T, cfg.E, device="cuda")
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, inp["X"], inp["W_r"], None, logits, plan, ws, nb)
    Xp = torch.full((plan.R_max, cfg.d), 7.0, dtype=torch.bfloat16, device="cuda")
    B.moe_permute(dims, plan, inp["X"], Xp)
    torch.cuda.synchronize()
    hp = plan.to_host()
    R = hp["R"]
    cnt = np.diff(hp["tok_off"])
    assert (cnt.max() > cfg.K) if round_mode == 2 else (cnt.min() == 0)
    want = inp["X"][torch.as_tensor(hp["row_token"], device="cuda").long()]
    assert torch.equal(Xp[:R].view(torch.int16), want.view(torch.int16))
    assert bool((Xp[R:] == 7.0).all())


def test_permute_packed_ffn_and_combine():
    cfg = wl.small_shape(T=600, d=192, E=6, K=3, n=128, dtype="bf16", seed=11)
    inp = wl.make_inputs(cfg, device="cuda")
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16")
    plan = B.Plan(dims)
    logits = torch.empty(cfg.T, cfg.E, device="cuda")
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, inp["X"], inp["W_r"], None, logits, plan, ws, nb)
    R_max = plan.R_max
    Xp = torch.zeros(R_max, cfg.d, dtype=torch.bfloat16, device="cuda")
    B.moe_permute(dims, plan, inp["X"], Xp)
    Yg = torch.empty(R_max, cfg.d, dtype=torch.bfloat16, device="cuda")
    Yp = torch.empty_like(Yg)
    Hg = torch.empty(R_max, 2 * cfg.n, dtype=torch.bfloat16, device="cuda")
    Hp = torch.empty_like(Hg)
    wsf, nbf = B.workspace(dims, B.OP_FFN)
    B.moe_grouped_ffn(dims, plan, inp["X"], True, inp["W_gate"], inp["W_up"], inp["W_down"], Hg, Yg, wsf, nbf)
    B.moe_grouped_ffn(dims, plan, Xp, False, inp["W_gate"], inp["W_up"], inp["W_down"], Hp, Yp, wsf, nbf)
    out_w = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
    out_u = torch.empty_like(out_w)
    B.moe_combine(dims, plan, Yg, True, out_w)
    B.moe_combine(dims, plan, Xp, False, out_u)
    torch.cuda.synchronize()
    hp = plan.to_host()
    R = hp["R"]
    # permute: bit-exact row copies; unpermute(permute(X)) is the replicated X
    X = inp["X"].cpu()
    assert torch.equal(Xp[:R].cpu(), X[torch.from_numpy(hp["row_token"]).long()])
    Z = oracle.unpermute(Xp[:R].cpu().view(torch.int16).numpy(), hp["tok_row"])
    rep = np.repeat(X.view(torch.int16).numpy(), np.diff(hp["tok_off"]), axis=0)
    assert np.array_equal(Z, rep)
    # packed and gathered inputs feed identical bits to the same GEMMs
    assert torch.equal(Yg[:R], Yp[:R]) and torch.equal(Hg[:R], Hp[:R])
    # weighted combine of the expert outputs = the layer output; unit combine of X_perm = K X
    ref = oracle.build_plan(f64(logits), cfg.K)
    fw = oracle.layer_forward(f64(inp["X"]), f64(inp["W_gate"]), f64(inp["W_up"]), f64(inp["W_down"]), ref)
    assert_close("out", f64(out_w), fw["out"], TOL["bf16"])
    assert_close("Y_perm", f64(Yg[:R]), fw["Y_perm"], TOL["bf16"])
    assert_close("unit combine", f64(out_u), cfg.K * f64(inp["X"]), TOL["bf16"])


@pytest.mark.parametrize("mode", [0, 1])
def test_route_nan_and_inf_logits(mode):
    """Non-finite logits still give K distinct experts per token and a valid permutation, with the
    same selection as the oracle (NaN ranks below every number, ties to the lower expert id)."""
    T, E, K = 500, 70, 6
    g = torch.Generator().manual_seed(7 + mode)
    L = torch.randn(T, E, generator=g)
    L[torch.rand(T, E, generator=g) < 0.2] = float("nan")
    L[torch.rand(T, E, generator=g) < 0.05] = float("inf")
    L[torch.rand(T, E, generator=g) < 0.05] = float("-inf")
    L[3, :] = float("nan")
    dims = B.make_dims(T, 64, 64, E, K, "f32", mode, 16)
    plan = B.Plan(dims)
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, None, None, None, L.cuda(), plan, ws, nb)
    torch.cuda.synchronize()
    got = plan.to_host()
    with np.errstate(invalid="ignore"):  # the softmax of a token with infinite logits
        ref = oracle.build_plan(L.double().numpy(), K, round_mode=mode, tile_m=16)
    for k in ("counts", "expert_off", "row_token", "tok_off", "tok_row"):
        assert np.array_equal(got[k], ref[k]), k
    assert np.array_equal(got["topk_idx"].reshape(T, K), ref["topk_idx"])
    idx = got["topk_idx"].reshape(T, K)
    assert all(len(set(r.tolist())) == K for r in idx)
    assert sorted(got["tok_row"].tolist()) == list(range(got["R"]))

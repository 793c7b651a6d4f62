"""The allocation-free routing entry point (moe_route_noalloc) against moe_route through the C ABI:
two calls in a row on one device, the second with a smaller layer, each giving bitwise the same
logits and plan as moe_route with a caller workspace (the same kernels; only the workspace
differs).  The first call needs most of the static buffer (token rounding keeps every logit key
there), the second reuses the buffer with stale contents from the first."""
import pytest
import torch

from conftest import announce_case
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl
from parity import dims_of

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


def route(cfg, inp, noalloc):
    dims = dims_of(cfg, inp["round_rand"])
    plan = B.Plan(dims)
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    if noalloc:
        B.moe_route_noalloc(dims, inp["X"], inp["W_r"], inp["bias"], logits, plan)
    else:
        ws, nb = B.workspace(dims, B.OP_ROUTE)
        B.moe_route(dims, inp["X"], inp["W_r"], inp["bias"], logits, plan, ws, nb)
    torch.cuda.synchronize()
    return logits, plan


def test_route_noalloc_matches_route_on_two_calls():
    # T and E of the Kimi-K2-shaped layer with token rounding to 128 (53 MiB of routing workspace)
    big = wl.small_shape(T=32768, d=512, E=384, K=8, n=64, dtype="bf16", bias="zipf", backward=False,
                         round_mode=1, tile_m=128, seed=80)
    small = wl.small_shape(T=1000, d=256, E=16, K=2, n=128, dtype="bf16", bias="normal", backward=False, seed=81)
    dims_big = dims_of(big)
    assert B.moe_workspace_bytes(dims_big, B.OP_ROUTE) > B.moe_route_noalloc_max_bytes() // 2
    for cfg in (big, small):
        inp = wl.make_inputs(cfg, device="cuda")
        L0, p0 = route(cfg, inp, noalloc=False)
        L1, p1 = route(cfg, inp, noalloc=True)
        assert torch.equal(L0, L1)
        h0, h1 = p0.to_host(), p1.to_host()
        R = h0["R"]
        assert h1["R"] == R
        for k in ("topk_idx", "topk_w", "counts", "expert_off", "tok_off"):
            assert (h0[k] == h1[k]).all(), k
        for k in ("row_token", "row_w", "tok_row"):
            assert (h0[k][:R] == h1[k][:R]).all(), k
        del inp

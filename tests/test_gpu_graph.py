"""The layer's forward and backward captured into a HIP graph and replayed.

The library's calls only enqueue kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a caller can capture moe_forward + moe_backward once and replay them.  Every
kernel of the path is deterministic, so each replay must reproduce the eager call bit for bit.
The replays are separated by eager work of the program's own and by synchronisations, and each
one is checked, with the outputs cleared in between so that a replay that wrote nothing fails.
"""
import pytest
import torch

from conftest import announce_case
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


def make_step(cfg, inp):
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, cfg.dtype, cfg.round_mode, cfg.tile_m,
                       inp["round_rand"])
    dt = B.torch_dtype(dims)
    plan = B.Plan(dims)
    R = plan.R_max
    f32 = dict(dtype=torch.float32, device="cuda")
    t = dict(logits=torch.empty(cfg.T, cfg.E, **f32), H=torch.empty(R, 2 * cfg.n, dtype=dt, device="cuda"),
             out=torch.empty(cfg.T, cfg.d, dtype=dt, device="cuda"), dX=torch.empty_like(inp["X"]),
             dW_gate=torch.empty_like(inp["W_gate"]), dW_up=torch.empty_like(inp["W_up"]),
             dW_down=torch.empty_like(inp["W_down"]), dS=torch.empty(R, **f32),
             dLogits=torch.empty(cfg.T, cfg.E, **f32), dW_r=torch.empty_like(inp["W_r"]))
    ws_f, nb_f = B.workspace(dims, B.OP_FORWARD)
    ws_b, nb_b = B.workspace(dims, B.OP_BACKWARD)

    def step():
        B.moe_forward(dims, inp["X"], inp["W_r"], inp["bias"], inp["W_gate"], inp["W_up"], inp["W_down"],
                      t["logits"], plan, t["H"], t["out"], ws_f, nb_f)
        B.moe_backward(dims, inp["dY"], inp["X"], inp["W_r"], inp["W_gate"], inp["W_up"], inp["W_down"],
                       plan, t["H"], t["dX"], t["dW_gate"], t["dW_up"], t["dW_down"], t["dS"], t["dLogits"],
                       t["dW_r"], ws_b, nb_b)

    outs = dict(t, row_token=plan.row_token, row_w=plan.row_w, expert_off=plan.expert_off, meta=plan.meta)
    return step, outs


@pytest.mark.parametrize("round_mode", [0, 1])
def test_forward_backward_graph_replays_match_eager(round_mode):
    cfg = wl.small_shape(T=700, d=320, E=6, K=2, n=192, dtype="bf16", backward=True, seed=23,
                         round_mode=round_mode, tile_m=64)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=True)
    step, outs = make_step(cfg, inp)
    step()
    torch.cuda.synchronize()
    names = ("logits", "out", "dX", "dW_gate", "dW_up", "dW_down", "dS", "dLogits", "dW_r",
             "row_token", "row_w", "expert_off", "meta")
    ref = {k: outs[k].clone() for k in names}
    R = int(ref["meta"][0].item())

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream's side, as torch asks before capturing
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for k in names:
            outs[k].fill_(0)
        noise = torch.randn(1 << 20, device="cuda").sum()  # the program's own eager work
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        for k in names:
            got, want = outs[k], ref[k]
            if k in ("row_token", "row_w", "dS"):
                got, want = got[:R], want[:R]
            assert torch.equal(got, want), "replay %d: %s differs from the eager call" % (rep, k)

"""GPU parity of the FP8 expert FFN (moe_quantize_fp8, moe_grouped_ffn_fp8) against the oracle.

Quantisation is a decision on exact values (power-of-two row scales make x / s exact), so codes
and scales are compared bit for bit, both for the inputs and -- fed the kernel's own bf16
activation -- for the activation.  The activation itself is compared with the oracle's exact
SwiGLU of the dequantised operands, and Y with the oracle's down product of the kernel's
activation codes, both within max|y - y_ref| <= 1e-2 max|y_ref| (fp32 sums of exact products,
one bf16 rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as F
from conftest import announce_case
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl
from parity import assert_close, f64

pytestmark = pytest.mark.gpu
TOL8 = 1e-2


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


def quantize(t):
    rows, K = t.reshape(-1, t.shape[-1]).shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, dtype=torch.float32, device="cuda")
    B.moe_quantize_fp8(t.reshape(rows, K), codes, scales)
    return codes, scales


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_matches_oracle(dtype):
    g = torch.Generator().manual_seed(5)
    X = torch.randn(67, 1544, generator=g) * torch.exp(torch.randn(67, 1, generator=g) * 4)
    X[3] = 0.0
    X[5, ::7] = -0.0
    X[9] = X[9] * 1e-30  # tiny rows: subnormal codes
    X[11, 0] = 448.0 * 2 ** 10
    Xt = X.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()
    codes, scales = quantize(Xt)
    torch.cuda.synchronize()
    ref_c, ref_s = F.quantize_rows(f64(Xt))
    assert np.array_equal(codes.cpu().numpy(), ref_c)
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref_s)


def test_quantize_ties_and_subnormals():
    """Rows whose elements sit exactly halfway between adjacent E4M3 values (normal and subnormal,
    both signs), just beside those midpoints, and on the codes themselves: the kernel's codes
    must be the oracle's (nearest, ties to the even code).  Each row's maximum is 448 times a
    power of two, so its scale is that power and every scaled value is exact."""
    grid = F.e4m3_decode(np.arange(0, 0x7F))
    mids = (grid[1:] + grid[:-1]) / 2
    m32 = mids.astype(np.float32)  # every midpoint is exact in fp32
    vals = np.concatenate([m32, grid.astype(np.float32), np.nextafter(m32, np.float32(0)),
                           np.nextafter(m32, np.float32(1e9))]).astype(np.float64)
    rows = []
    for sgn in (1.0, -1.0):
        for p2 in (0, -20, 7):
            r = np.concatenate([[448.0], sgn * vals]) * 2.0 ** p2
            rows.append(np.resize(r, 512))
    X = torch.tensor(np.array(rows), dtype=torch.float32).cuda()
    codes, scales = quantize(X)
    torch.cuda.synchronize()
    ref_c, ref_s = F.quantize_rows(f64(X))
    assert np.array_equal(scales.cpu().numpy().astype(np.float64), ref_s)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, [(int(i), int(j), float(f64(X)[i, j]), int(got[i, j]), int(ref_c[i, j])) for i, j in bad[:8]]


def run_ffn_fp8(cfg, inp):
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16")
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    plan = B.Plan(dims)
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, inp["X"], inp["W_r"], inp["bias"], logits, plan, ws, nb)
    Xq, sx = quantize(inp["X"])
    Wgq, sg = quantize(inp["W_gate"].reshape(-1, cfg.d))
    Wuq, su = quantize(inp["W_up"].reshape(-1, cfg.d))
    Wdq, sd = quantize(inp["W_down"].reshape(-1, cfg.n))
    R = B.moe_max_rows(dims)
    act = torch.empty(R, cfg.n, dtype=torch.bfloat16, device="cuda")
    act_q = torch.empty(R, cfg.n, dtype=torch.uint8, device="cuda")
    sact = torch.empty(R, dtype=torch.float32, device="cuda")
    Y = torch.empty(R, cfg.d, dtype=torch.bfloat16, device="cuda")
    wsf, nbf = B.workspace(dims, B.OP_FFN_FP8)
    B.moe_grouped_ffn_fp8(dims, plan, Xq, sx, Wgq, sg, Wuq, su, Wdq, sd, act, act_q, sact, Y, wsf, nbf)
    torch.cuda.synchronize()
    return dict(logits=logits, plan=plan, Xq=Xq, sx=sx, Wgq=Wgq.reshape(cfg.E, cfg.n, cfg.d), sg=sg.reshape(cfg.E, cfg.n),
                Wuq=Wuq.reshape(cfg.E, cfg.n, cfg.d), su=su.reshape(cfg.E, cfg.n), Wdq=Wdq.reshape(cfg.E, cfg.d, cfg.n),
                sd=sd.reshape(cfg.E, cfg.d), act=act, act_q=act_q, sact=sact, Y=Y)


def check_ffn_fp8(cfg, inp, out, experts):
    plan_ref = oracle.build_plan(f64(out["logits"]), cfg.K)
    off = out["plan"].expert_off.cpu().numpy()
    tok = out["plan"].row_token.cpu().numpy()
    assert np.array_equal(off, plan_ref["expert_off"]) and np.array_equal(tok[:off[-1]], plan_ref["row_token"])
    # inputs: codes and scales bit-exact
    ref_xc, ref_xs = F.quantize_rows(f64(inp["X"]))
    assert np.array_equal(out["Xq"].cpu().numpy(), ref_xc) and np.array_equal(out["sx"].cpu().numpy(), ref_xs)
    Xq, sx = out["Xq"].cpu().numpy(), out["sx"].cpu().numpy().astype(np.float64)
    act = out["act"]
    worst = {}
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        # every weight operand's codes and scales bit-exact against the oracle's quantisation
        for w, q, sc in (("W_gate", "Wgq", "sg"), ("W_up", "Wuq", "su"), ("W_down", "Wdq", "sd")):
            c_ref, s_ref = F.quantize_rows(f64(inp[w][e]))
            assert np.array_equal(out[q][e].cpu().numpy(), c_ref), "%s codes e%d" % (w, e)
            assert np.array_equal(out[sc][e].cpu().numpy(), s_ref), "%s scales e%d" % (w, e)
        Wgq = {e: out["Wgq"][e].cpu().numpy()}
        Wuq = {e: out["Wuq"][e].cpu().numpy()}
        sg = {e: out["sg"][e].cpu().numpy().astype(np.float64)}
        su = {e: out["su"][e].cpu().numpy().astype(np.float64)}
        _, _, A = F.ffn_fp8_up(Xq, sx, Wgq, sg, Wuq, su, tok, off, e)
        a_gpu = f64(act[r0:r1])
        worst["act"] = max(worst.get("act", 0), assert_close("act e%d" % e, a_gpu, A, TOL8))
        ac, asc = F.quantize_rows(a_gpu)
        assert np.array_equal(out["act_q"][r0:r1].cpu().numpy(), ac), "act codes e%d" % e
        assert np.array_equal(out["sact"][r0:r1].cpu().numpy().astype(np.float64), asc), "act scales e%d" % e
        Aq = np.zeros((int(off[-1]), cfg.n), np.uint8)
        sa = np.ones(int(off[-1]))
        Aq[r0:r1], sa[r0:r1] = ac, asc
        Y = F.ffn_fp8_down(Aq, sa, {e: out["Wdq"][e].cpu().numpy()}, {e: out["sd"][e].cpu().numpy().astype(np.float64)},
                           off, e)
        worst["Y"] = max(worst.get("Y", 0), assert_close("Y e%d" % e, f64(out["Y"][r0:r1]), Y, TOL8))
    return worst


# d <= 2048 runs the gate/up GEMM and n <= 2048 the down GEMM on the half-width engine; d or n =
# 2112 takes the four-wave one
@pytest.mark.parametrize("T,d,n,E,K", [(700, 320, 192, 6, 2), (129, 256, 64, 4, 4), (1000, 512, 320, 8, 2),
                                       (300, 192, 2112, 4, 2), (200, 2112, 128, 3, 2)])
def test_grouped_ffn_fp8_small(T, d, n, E, K):
    cfg = wl.small_shape(T=T, d=d, E=E, K=K, n=n, dtype="bf16", backward=False, seed=T + d)
    inp = wl.make_inputs(cfg, device="cuda")
    out = run_ffn_fp8(cfg, inp)
    print(check_ffn_fp8(cfg, inp, out, range(E)))


@pytest.mark.slow
def test_grouped_ffn_fp8_fine_grained_sampled():
    cfg = wl.BY_NAME["fine_grained_7b"].with_(backward=False)
    inp = wl.make_inputs(cfg, device="cuda")
    out = run_ffn_fp8(cfg, inp)
    print(check_ffn_fp8(cfg, inp, out, [0, 57, 127]))

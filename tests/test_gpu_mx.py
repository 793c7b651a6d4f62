"""GPU parity of the block-scaled FP8 expert FFN (moe_quantize_mx, moe_grouped_ffn_mx) against
oracle/mx.py, in both element formats (E4M3 and E5M2).

Quantisation is a decision on exact values (a power-of-two block scale makes x / s exact), so codes
and scale bytes are compared bit for bit: for the inputs, and -- fed the kernel's own bf16
activation, which the gate/up GEMM returns beside its codes -- for the activation quantised in
that GEMM's epilogue.  The activation is compared with the oracle's exact SwiGLU of the
dequantised operands, and Y with the oracle's down product of the kernel's activation codes, both
within max|y - y_ref| <= 1e-2 max|y_ref| (fp32 sums of exact block products, one bf16 rounding).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mx as M
from conftest import announce_case
from mixture_experts_layer_lds_amd import binding as B
from mixture_experts_layer_lds_amd import workloads as wl
from parity import assert_close, f64

pytestmark = pytest.mark.gpu
TOL8 = 1e-2
FMT = {B.FP8_E4M3: "e4m3", B.FP8_E5M2: "e5m2"}


@pytest.fixture(autouse=True)
def announce(request):
    announce_case(request.node.nodeid)
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    yield
    torch.cuda.empty_cache()


def quantize(t, fmt):
    t = t.reshape(-1, t.shape[-1])
    rows, K = t.shape
    codes = torch.empty(rows, K, dtype=torch.uint8, device="cuda")
    scales = torch.empty(B.moe_mx_scale_bytes(rows, K), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mx(t, fmt, codes, scales)
    return codes, scales


def by_row(scales, rows, K):
    """The library's group-major block scales (byte (b / 4) * rows * 4 + r * 4 + b % 4 for block b
    of row r) as a [rows, K / 32] array, the oracle's layout."""
    g = (K + 127) // 128
    a = scales.reshape(-1).cpu().numpy()[:g * rows * 4].reshape(g, rows, 4)
    return a.transpose(1, 0, 2).reshape(rows, 4 * g)[:, :K // 32]


@pytest.mark.parametrize("fmt", [B.FP8_E4M3, B.FP8_E5M2])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_quantize_mx_matches_oracle(fmt, dtype):
    """Random blocks over a wide dynamic range, an all-zero block, signed zeros, a block of tiny
    values (scale near 2^-100), a block whose maximum is the format's largest value, and K = 1600
    (50 blocks: the scale stride has padding)."""
    g = torch.Generator().manual_seed(7 + fmt)
    K = 1600
    X = torch.randn(53, K, generator=g) * torch.exp(torch.randn(53, K // 32, generator=g) * 5).repeat_interleave(32, 1)
    X[3, 64:96] = 0.0
    X[5, ::7] = -0.0
    X[9, :32] = X[9, :32] * 1e-30
    X[11, 32] = M.max_finite(FMT[fmt])
    Xt = X.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()
    codes, scales = quantize(Xt, fmt)
    torch.cuda.synchronize()
    ref_c, ref_s = M.quantize_blocks(f64(Xt), FMT[fmt])
    assert np.array_equal(by_row(scales, Xt.shape[0], K), ref_s)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, [(int(i), int(j), float(f64(Xt)[i, j]), int(got[i, j]), int(ref_c[i, j])) for i, j in bad[:8]]


@pytest.mark.parametrize("fmt", [B.FP8_E4M3, B.FP8_E5M2])
def test_quantize_mx_ties(fmt):
    """Blocks whose values sit exactly halfway between adjacent codes (normal and subnormal, both
    signs), just beside those midpoints, and on the codes themselves; each block's maximum is the
    format's largest value times a power of two, so the block scale is that power and every scaled
    value is exact: the kernel's codes must be the oracle's (nearest, ties to the even code)."""
    name = FMT[fmt]
    top = 0x7E if name == "e4m3" else 0x7B
    grid = M.decode(np.arange(0, top + 1), name)
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    vals = np.concatenate([mids, grid.astype(np.float32), np.nextafter(mids, np.float32(0)),
                           np.nextafter(mids, np.float32(1e9))]).astype(np.float64)
    nblk = int(np.ceil(len(vals) / 31))
    rows = []
    for sgn in (1.0, -1.0):
        for p2 in (0, -20, 7):
            r = np.zeros(nblk * 32)
            for b in range(nblk):
                chunk = vals[31 * b:31 * (b + 1)]
                r[32 * b] = M.max_finite(name)
                r[32 * b + 1:32 * b + 1 + len(chunk)] = sgn * chunk
            rows.append(r * 2.0 ** p2)
    K = (nblk * 32 + 63) // 64 * 64
    X = torch.zeros(len(rows), K, dtype=torch.float32)
    X[:, :nblk * 32] = torch.tensor(np.array(rows), dtype=torch.float32)
    X = X.cuda()
    codes, scales = quantize(X, fmt)
    torch.cuda.synchronize()
    ref_c, ref_s = M.quantize_blocks(f64(X), name)
    assert np.array_equal(by_row(scales, X.shape[0], K), ref_s)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != ref_c)
    assert bad.size == 0, [(int(i), int(j), float(f64(X)[i, j]), int(got[i, j]), int(ref_c[i, j])) for i, j in bad[:8]]


def run_ffn_mx(cfg, inp, fmt):
    dims = B.make_dims(cfg.T, cfg.d, cfg.n, cfg.E, cfg.K, "bf16")
    logits = torch.empty(cfg.T, cfg.E, dtype=torch.float32, device="cuda")
    plan = B.Plan(dims)
    ws, nb = B.workspace(dims, B.OP_ROUTE)
    B.moe_route(dims, inp["X"], inp["W_r"], inp["bias"], logits, plan, ws, nb)
    Xq, sx = quantize(inp["X"], fmt)
    Wgq, sg = quantize(inp["W_gate"], fmt)
    Wuq, su = quantize(inp["W_up"], fmt)
    Wdq, sd = quantize(inp["W_down"], fmt)
    R = B.moe_max_rows(dims)
    act = torch.empty(R, cfg.n, dtype=torch.bfloat16, device="cuda")
    act_q = torch.empty(R, cfg.n, dtype=torch.uint8, device="cuda")
    sact = torch.empty(B.moe_mx_scale_bytes(R, cfg.n), dtype=torch.uint8, device="cuda")
    Y = torch.empty(R, cfg.d, dtype=torch.bfloat16, device="cuda")
    wsf, nbf = B.workspace(dims, B.OP_FFN_MX)
    B.moe_grouped_ffn_mx(dims, plan, fmt, Xq, sx, Wgq, sg, Wuq, su, Wdq, sd, act, act_q, sact, Y, wsf, nbf)
    torch.cuda.synchronize()
    E, n, d = cfg.E, cfg.n, cfg.d
    return dict(logits=logits, plan=plan, R_max=R, Xq=Xq, sx=by_row(sx, cfg.T, d), Wgq=Wgq.reshape(E, n, d),
                sg=by_row(sg, E * n, d).reshape(E, n, -1), Wuq=Wuq.reshape(E, n, d),
                su=by_row(su, E * n, d).reshape(E, n, -1), Wdq=Wdq.reshape(E, d, n),
                sd=by_row(sd, E * d, n).reshape(E, d, -1), act=act, act_q=act_q, sact=by_row(sact, R, n), Y=Y)


def sample_rows(r0, r1, max_rows):
    """Rows r0 .. r1 - 1 of an expert, or max_rows of them spread evenly (first and last kept)."""
    if max_rows is None or r1 - r0 <= max_rows:
        return np.arange(r0, r1)
    return np.unique(np.linspace(r0, r1 - 1, max_rows).round().astype(np.int64))


def check_ffn_mx(cfg, inp, out, experts, fmt, max_rows=None):
    """Codes and scales of X and of every checked expert's weights bit for bit; then, on the
    expert's rows (or max_rows of them), the activation, its codes and scales, and Y."""
    name = FMT[fmt]
    d, n = cfg.d, cfg.n
    plan_ref = oracle.build_plan(f64(out["logits"]), cfg.K)
    off = out["plan"].expert_off.cpu().numpy()
    tok = out["plan"].row_token.cpu().numpy()
    assert np.array_equal(off, plan_ref["expert_off"]) and np.array_equal(tok[:off[-1]], plan_ref["row_token"])
    ref_xc, ref_xs = M.quantize_blocks(f64(inp["X"]), name)
    assert np.array_equal(out["Xq"].cpu().numpy(), ref_xc) and np.array_equal(out["sx"], ref_xs)
    Xq, sx = out["Xq"].cpu().numpy(), out["sx"]
    worst = {}
    for e in experts:
        r0, r1 = int(off[e]), int(off[e + 1])
        w = {}
        for wn, q, sc, K in (("W_gate", "Wgq", "sg", d), ("W_up", "Wuq", "su", d), ("W_down", "Wdq", "sd", n)):
            c_ref, s_ref = M.quantize_blocks(f64(inp[wn][e]), name)
            c, s = out[q][e].cpu().numpy(), out[sc][e]
            assert np.array_equal(c, c_ref), "%s codes e%d" % (wn, e)
            assert np.array_equal(s, s_ref), "%s scales e%d" % (wn, e)
            w[q], w[sc] = {e: c}, {e: s}
        if r1 == r0:
            continue
        rows = sample_rows(r0, r1, max_rows)
        # the sampled rows as a one-expert plan (expert e renumbered 0)
        sub_off = np.array([0, len(rows)])
        sub = {k: {0: v[e]} for k, v in w.items()}
        idx = torch.from_numpy(rows).to(out["act"].device)
        _, _, A = M.ffn_mx_up(Xq, sx, sub["Wgq"], sub["sg"], sub["Wuq"], sub["su"], tok[rows], sub_off, 0, name)
        a_gpu = f64(out["act"].index_select(0, idx))
        worst["act"] = max(worst.get("act", 0), assert_close("act e%d" % e, a_gpu, A, TOL8))
        ac, asc = M.quantize_blocks(a_gpu, name)
        assert np.array_equal(out["act_q"].index_select(0, idx).cpu().numpy(), ac), "act codes e%d" % e
        assert np.array_equal(out["sact"][rows], asc), "act scales e%d" % e
        Y = M.ffn_mx_down(ac, asc, sub["Wdq"], sub["sd"], sub_off, 0, name)
        worst["Y"] = max(worst.get("Y", 0), assert_close("Y e%d" % e, f64(out["Y"].index_select(0, idx)), Y, TOL8))
    return worst


# d <= 2048 runs the gate/up GEMM and n <= 2048 the down GEMM on the half-width engine, d or n =
# 2112 (an odd number of 64-wide k-stages) on the four-wave one; there n = 192 leaves the last
# 128-column gate/up tile half empty and d = 192 the down tile's last 64 columns; n = 64 gives a
# scale stride with padding
@pytest.mark.parametrize("fmt", [B.FP8_E4M3, B.FP8_E5M2])
@pytest.mark.parametrize("T,d,n,E,K", [(700, 320, 192, 6, 2), (129, 256, 64, 4, 4), (1000, 512, 320, 8, 2),
                                       (300, 192, 2112, 4, 2), (200, 2112, 128, 3, 2), (260, 2112, 192, 3, 2)])
def test_grouped_ffn_mx_small(T, d, n, E, K, fmt):
    cfg = wl.small_shape(T=T, d=d, E=E, K=K, n=n, dtype="bf16", backward=False, seed=T + d + fmt)
    inp = wl.make_inputs(cfg, device="cuda")
    out = run_ffn_mx(cfg, inp, fmt)
    print(check_ffn_mx(cfg, inp, out, range(E), fmt))


@pytest.mark.slow
@pytest.mark.parametrize("fmt", [B.FP8_E4M3, B.FP8_E5M2])
def test_grouped_ffn_mx_fine_grained_sampled(fmt):
    """The fine-grained layer (T=32768, d=1536, E=128, K=8, n=256) in the launch configuration
    the benchmark times; experts 0, 57 and 127 compared."""
    cfg = wl.BY_NAME["fine_grained_7b"].with_(backward=False)
    inp = wl.make_inputs(cfg, device="cuda")
    out = run_ffn_mx(cfg, inp, fmt)
    print(check_ffn_mx(cfg, inp, out, [0, 57, 127], fmt))


@pytest.mark.slow
def test_grouped_ffn_mx_mixtral_sampled():
    """The coarse layer (T=8192, d=4096, n=14336, E=8, K=2): both GEMMs on the four-wave engine
    (K = 4096 and 14336); experts 0 and 7, 48 rows of each."""
    cfg = wl.BY_NAME["mixtral_coarse"].with_(backward=False)
    inp = wl.make_inputs(cfg, device="cuda")
    out = run_ffn_mx(cfg, inp, B.FP8_E4M3)
    print(check_ffn_mx(cfg, inp, out, [0, 7], B.FP8_E4M3, max_rows=48))

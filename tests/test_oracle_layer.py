"""Pins of the oracle's layer forward and backward against independent computations.

* forward against a dense brute force: every expert evaluated on every token (torch float64,
  ``torch.nn.functional.silu``), masked to the token's final experts and weighted by a masked
  softmax; special cases E=1/K=1 (a plain SwiGLU FFN), identical experts (FFN(x) whatever the
  routing) and K=E (the full softmax mixture);
* backward against torch autograd of that dense formulation (routing held fixed) and against
  central finite differences of the oracle's own forward;
* the router-score identity <dY_t, Y_{t,e}> = <dY_t Wd_e, A_{t,e}> (SonicMoE page, dS row of the
  kernel table) and the softmax-Jacobian property sum_j dLogits[t, j] = 0.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import softmax

import oracle


def rand_layer(seed, T, d, E, n, bias=True):
    rng = np.random.default_rng(seed)
    return dict(
        X=rng.normal(size=(T, d)),
        W_r=rng.normal(size=(E, d)) * 0.5,
        bias=rng.normal(size=E) if bias else None,
        Wg=rng.normal(size=(E, n, d)) / np.sqrt(d),
        Wu=rng.normal(size=(E, n, d)) / np.sqrt(d),
        Wd=rng.normal(size=(E, d, n)) / np.sqrt(n),
        dY=rng.normal(size=(T, d)),
    )


def dense_torch(p, sel, requires_grad=False):
    """All experts on all tokens, masked softmax weights; returns (out, logits, leaf tensors)."""
    leaves = {k: torch.tensor(p[k], dtype=torch.float64, requires_grad=requires_grad)
              for k in ("X", "W_r", "Wg", "Wu", "Wd")}
    X, W_r, Wg, Wu, Wd = (leaves[k] for k in ("X", "W_r", "Wg", "Wu", "Wd"))
    L = X @ W_r.T
    if p["bias"] is not None:
        L = L + torch.tensor(p["bias"], dtype=torch.float64)
    if requires_grad:
        L.retain_grad()
    mask = torch.tensor(sel)
    w = torch.softmax(L.masked_fill(~mask, float("-inf")), dim=1)
    w = torch.where(mask.any(dim=1, keepdim=True), w, torch.zeros_like(w))
    out = torch.zeros_like(X)
    for e in range(Wg.shape[0]):
        Y = (F.silu(X @ Wg[e].T) * (X @ Wu[e].T)) @ Wd[e].T
        out = out + w[:, e:e + 1] * Y
    return out, L, leaves


def oracle_plan(p, K, mode=0, M=4):
    L = oracle.router_logits(p["X"], p["W_r"], p["bias"])
    return L, oracle.build_plan(L, K, round_mode=mode, tile_m=M)


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
@pytest.mark.parametrize("K", [1, 2, 3])
def test_forward_matches_dense_bruteforce(mode, K):
    p = rand_layer(10 * K + mode, T=37, d=12, E=5, n=10)
    L, plan = oracle_plan(p, K, mode)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    ref, _, _ = dense_torch(p, plan["sel"])
    assert np.allclose(fw["out"], ref.numpy(), rtol=0, atol=1e-12)
    # permuted-layout intermediates are the per-row expert outputs
    for r in range(0, len(plan["row_token"]), 7):
        t, e = plan["row_token"][r], plan["row_expert"][r]
        x = torch.tensor(p["X"][t])
        G = x @ torch.tensor(p["Wg"][e]).T
        U = x @ torch.tensor(p["Wu"][e]).T
        Y = (F.silu(G) * U) @ torch.tensor(p["Wd"][e]).T
        assert np.allclose(fw["Y_perm"][r], Y.numpy(), atol=1e-12)
        assert np.allclose(fw["H"][r], np.concatenate([G.numpy(), U.numpy()]), atol=1e-12)
    tf = oracle.token_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan, [0, 5, 36])
    assert np.allclose(tf, fw["out"][[0, 5, 36]], atol=1e-12)


def test_single_expert_is_dense_swiglu_ffn():
    p = rand_layer(1, T=9, d=16, E=1, n=24, bias=False)
    L, plan = oracle_plan(p, 1)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    x = torch.tensor(p["X"])
    ffn = (F.silu(x @ torch.tensor(p["Wg"][0]).T) * (x @ torch.tensor(p["Wu"][0]).T)) \
        @ torch.tensor(p["Wd"][0]).T
    assert np.allclose(fw["out"], ffn.numpy(), rtol=0, atol=1e-12)
    assert np.all(plan["row_w"] == 1.0)


@pytest.mark.parametrize("K", [1, 3, 6])
def test_identical_experts_give_ffn_for_any_routing(K):
    p = rand_layer(2, T=20, d=8, E=6, n=12)
    for k in ("Wg", "Wu", "Wd"):
        p[k] = np.repeat(p[k][:1], 6, axis=0)
    L, plan = oracle_plan(p, K)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    x = torch.tensor(p["X"])
    ffn = (F.silu(x @ torch.tensor(p["Wg"][0]).T) * (x @ torch.tensor(p["Wu"][0]).T)) \
        @ torch.tensor(p["Wd"][0]).T
    assert np.allclose(fw["out"], ffn.numpy(), rtol=0, atol=1e-12)


def test_all_experts_is_full_softmax_mixture():
    p = rand_layer(3, T=15, d=8, E=4, n=6)
    L, plan = oracle_plan(p, 4)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    w = softmax(L, axis=1)
    ref = np.zeros_like(p["X"])
    for e in range(4):
        G = p["X"] @ p["Wg"][e].T
        ref += w[:, e:e + 1] * ((G * softmax(np.stack([np.zeros_like(G), G]), axis=0)[1]
                                 * (p["X"] @ p["Wu"][e].T)) @ p["Wd"][e].T)
    assert np.allclose(fw["out"], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("mode", [0, 1, 3])
def test_backward_matches_autograd(mode):
    p = rand_layer(40 + mode, T=33, d=10, E=6, n=8)
    L, plan = oracle_plan(p, 2, mode, M=4)
    bw = oracle.layer_backward(p["dY"], p["X"], p["Wg"], p["Wu"], p["Wd"], plan, W_r=p["W_r"])
    out, Lt, leaves = dense_torch(p, plan["sel"], requires_grad=True)
    (out * torch.tensor(p["dY"])).sum().backward()
    tol = dict(rtol=1e-10, atol=1e-11)
    assert np.allclose(bw["dX"], leaves["X"].grad.numpy(), **tol)
    assert np.allclose(bw["dW_r"], leaves["W_r"].grad.numpy(), **tol)
    assert np.allclose(bw["dLogits"], Lt.grad.numpy(), **tol)
    for e in range(6):
        assert np.allclose(bw["dW_gate"][e], leaves["Wg"].grad[e].numpy(), **tol)
        assert np.allclose(bw["dW_up"][e], leaves["Wu"].grad[e].numpy(), **tol)
        assert np.allclose(bw["dW_down"][e], leaves["Wd"].grad[e].numpy(), **tol)


def test_router_score_identity_and_jacobian_rows():
    p = rand_layer(7, T=40, d=12, E=8, n=16)
    L, plan = oracle_plan(p, 3)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    bw = oracle.layer_backward(p["dY"], p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    direct = np.einsum("rd,rd->r", p["dY"][plan["row_token"]], fw["Y_perm"])
    assert np.allclose(bw["dS"], direct, rtol=0, atol=1e-12)
    assert np.allclose(bw["dLogits"].sum(axis=1), 0.0, atol=1e-14)
    assert np.all(bw["dLogits"][~plan["sel"]] == 0.0)


def test_backward_matches_finite_differences():
    """Central differences of the oracle's forward (selection frozen, weights recomputed)."""
    p = rand_layer(8, T=4, d=8, E=4, n=8)
    L0, plan0 = oracle_plan(p, 2)
    sel = plan0["sel"]

    def loss(q):
        L = oracle.router_logits(q["X"], q["W_r"], q["bias"])
        W = oracle.gate_weights(L, sel)
        plan = dict(plan0, row_w=W[plan0["row_token"], plan0["row_expert"]])
        out = oracle.layer_forward(q["X"], q["Wg"], q["Wu"], q["Wd"], plan)["out"]
        return float(np.sum(out * q["dY"]))

    bw = oracle.layer_backward(p["dY"], p["X"], p["Wg"], p["Wu"], p["Wd"], plan0, W_r=p["W_r"])
    grads = dict(X=bw["dX"], W_r=bw["dW_r"],
                 Wg=np.stack([bw["dW_gate"][e] for e in range(4)]),
                 Wu=np.stack([bw["dW_up"][e] for e in range(4)]),
                 Wd=np.stack([bw["dW_down"][e] for e in range(4)]))
    rng = np.random.default_rng(0)
    h = 1e-6
    for name, g in grads.items():
        for _ in range(6):
            idx = tuple(rng.integers(0, s) for s in p[name].shape)
            q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
            q[name][idx] += h
            up = loss(q)
            q[name][idx] -= 2 * h
            dn = loss(q)
            fd = (up - dn) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])


@pytest.mark.parametrize("mode", [0, 1])
def test_weighted_combine_is_the_dense_mixture(mode):
    """The weighted branch of ``oracle.combine`` (per token, rows in ascending expert, each scaled
    by its gate weight) applied to the experts' outputs Y_perm equals the dense brute force (every
    expert on every token, masked softmax weights), with and without token rounding; and a hand
    example with distinct weights."""
    p = rand_layer(40 + mode, T=11, d=6, E=5, n=7)
    L, plan = oracle_plan(p, K=2, mode=mode, M=4)
    fw = oracle.layer_forward(p["X"], p["Wg"], p["Wu"], p["Wd"], plan)
    out = oracle.combine(fw["Y_perm"], plan["tok_off"], plan["tok_row"], plan["row_w"])
    dense, _, _ = dense_torch(p, plan["sel"])
    assert np.allclose(out, dense.numpy(), rtol=0, atol=1e-12)
    # hand example: token 0 owns rows 0 and 2, token 1 row 1, token 2 none
    Y = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    got = oracle.combine(Y, np.array([0, 2, 3, 3]), np.array([0, 2, 1]), np.array([0.25, 0.5, 0.75]))
    assert np.array_equal(got, np.array([[4.0, 5.0], [1.5, 2.0], [0.0, 0.0]]))

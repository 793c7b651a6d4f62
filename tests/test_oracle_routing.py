"""Pins of the oracle's routing against things other than itself.

* top-K against a brute-force rank count (pairwise comparisons, no sorting);
* gate weights against the full softmax renormalised over the selection, and sum-to-one;
* token rounding against exhaustive subset enumeration on tiny inputs, plus its invariants
  (SonicMoE summary page, optimization 3: counts become tile multiples, at most one tile away);
* counts against the ThunderEP article's worked examples (sections 1 and 2.1);
* permutation indices against their defining identities.
"""
import itertools
import json
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_rank(L_row):
    """rank[e] = number of experts beating e under (logit desc, id asc) — O(E^2) comparisons."""
    E = len(L_row)
    rank = np.zeros(E, np.int64)
    for e in range(E):
        for f in range(E):
            if L_row[f] > L_row[e] or (L_row[f] == L_row[e] and f < e):
                rank[e] += 1
    return rank


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_bruteforce_rank_with_ties(seed):
    rng = np.random.default_rng(seed)
    T, E = 40, 9
    # small integer logits force many exact ties; include +0.0 / -0.0 which compare equal
    L = rng.integers(-3, 4, size=(T, E)).astype(np.float64)
    L[0, :] = 0.0
    L[1, ::2] = -0.0
    for K in (1, 2, 5, E):
        idx = oracle.topk_select(L, K)
        for t in range(T):
            rank = brute_rank(L[t])
            expect = np.array([int(np.nonzero(rank == j)[0][0]) for j in range(K)])
            assert np.array_equal(idx[t], expect), (t, K, L[t], idx[t], expect)


def test_weights_are_renormalised_full_softmax_and_sum_to_one():
    rng = np.random.default_rng(3)
    T, E, K = 64, 16, 4
    L = rng.normal(size=(T, E)) * 3
    plan = oracle.build_plan(L, K)
    full = softmax(L, axis=1)
    for t in range(T):
        es = plan["topk_idx"][t]
        ren = full[t, es] / full[t, es].sum()
        assert np.allclose(plan["topk_w"][t], ren, rtol=0, atol=1e-15)
        assert abs(plan["topk_w"][t].sum() - 1.0) < 1e-15
        assert np.allclose(plan["weights"][t, es], ren, rtol=0, atol=1e-15)
    assert np.array_equal(plan["weights"] > 0, plan["sel"])


def test_thunderep_count_examples():
    with open(os.path.join(GOLDEN, "thunderep_routing_counts.json")) as f:
        g = json.load(f)
    sp = g["split_example"]
    rng = np.random.default_rng(0)
    target = np.repeat(np.arange(sp["experts"]), sp["counts"])
    rng.shuffle(target)
    L = rng.normal(size=(sp["tokens"], sp["experts"])) * 0.1
    L[np.arange(sp["tokens"]), target] += 5.0
    plan = oracle.build_plan(L, sp["k"])
    assert plan["counts"].tolist() == sp["counts"]
    assert int(plan["expert_off"][-1]) == sp["tokens"]

    pe = g["pairs_example"]
    L = rng.normal(size=(pe["tokens"], pe["experts"]))
    plan = oracle.build_plan(L, pe["k"])
    assert int(plan["counts"].sum()) == pe["pairs"] == len(plan["row_token"])
    assert np.array_equal(plan["expert_off"], np.concatenate([[0], np.cumsum(plan["counts"])]))


def check_plan_identities(plan, T, E):
    R = int(plan["expert_off"][-1])
    rt, re_, tr = plan["row_token"], plan["row_expert"], plan["tok_row"]
    assert len(rt) == R == len(tr) == int(plan["tok_off"][-1])
    assert sorted(tr.tolist()) == list(range(R))               # bijection onto rows
    for e in range(E):                                          # segments sorted by token
        seg = rt[plan["expert_off"][e]:plan["expert_off"][e + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(re_[plan["expert_off"][e]:plan["expert_off"][e + 1]] == e)
    for t in range(T):
        rows = tr[plan["tok_off"][t]:plan["tok_off"][t + 1]]
        assert np.all(rt[rows] == t)
        assert np.all(np.diff(re_[rows]) > 0)                   # ascending expert
        assert set(re_[rows].tolist()) == set(np.nonzero(plan["sel"][t])[0].tolist())


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_permutation_identities(mode):
    rng = np.random.default_rng(11 + mode)
    T, E, K, d = 50, 7, 3, 5
    L = rng.normal(size=(T, E))
    plan = oracle.build_plan(L, K, round_mode=mode, tile_m=4)
    check_plan_identities(plan, T, E)
    X = rng.normal(size=(T, d)).astype(np.float32)
    Xp = oracle.permute(X, plan["row_token"])
    Z = oracle.unpermute(Xp, plan["tok_row"])
    rep = np.repeat(X, np.diff(plan["tok_off"]), axis=0)
    assert Z.dtype == X.dtype and np.array_equal(Z.view(np.uint32), rep.view(np.uint32))
    unit = oracle.combine(Xp, plan["tok_off"], plan["tok_row"])
    assert np.allclose(unit, np.diff(plan["tok_off"])[:, None] * X.astype(np.float64), atol=1e-12)
    if mode == 0:
        assert int(plan["counts"].sum()) == T * K


def pref_rank(col):
    """Position of each token in an expert's preference order (logit desc, token asc), by counting."""
    T = len(col)
    return np.array([sum(1 for u in range(T) if col[u] > col[t] or (col[u] == col[t] and u < t))
                     for t in range(T)])


def brute_round_expert(col, member, M, mode, T, word=None):
    """Exhaustive token rounding for one expert: target count, then best subset by enumeration.
    Stochastic mode: round up iff the word, read as the exact fraction word / 2^32, is below
    (c mod M) / M."""
    from fractions import Fraction
    c = int(member.sum())
    lower, upper = (c // M) * M, (c // M) * M + M
    if c % M == 0:
        target = c
    elif mode == 1:
        target = upper if 2 * (c - lower) >= M else lower
    elif mode == 2:
        target = upper
    elif mode == 4:
        target = upper if Fraction(int(word), 2 ** 32) < Fraction(c - lower, M) else lower
    else:
        target = lower
    if target > T:
        target = lower
    rank = pref_rank(col)
    mem = [t for t in range(T) if member[t]]
    non = [t for t in range(T) if not member[t]]
    new = member.copy()
    if target > c:      # add the subset of non-members with the smallest total rank
        best = min(itertools.combinations(non, target - c), key=lambda s: sum(rank[list(s)]))
        new[list(best)] = True
    elif target < c:    # drop the subset of members with the largest total rank
        best = max(itertools.combinations(mem, c - target), key=lambda s: sum(rank[list(s)]))
        new[list(best)] = False
    return new, target


@pytest.mark.parametrize("mode", [1, 2, 3, 4])
@pytest.mark.parametrize("M", [2, 3, 4])
@pytest.mark.parametrize("seed", range(4))
def test_token_rounding_matches_enumeration(mode, M, seed):
    rng = np.random.default_rng(100 * seed + 10 * M + mode)
    T, E, K = 9, 4, 2
    L = rng.integers(-2, 3, size=(T, E)).astype(np.float64)    # ties on purpose
    sel = np.zeros((T, E), bool)
    np.put_along_axis(sel, oracle.topk_select(L, K), True, axis=1)
    words = rng.integers(0, 2 ** 32, size=E, dtype=np.uint64).astype(np.uint32)
    got = oracle.token_rounding(L, sel, M, mode, words if mode == 4 else None)
    for e in range(E):
        exp_col, target = brute_round_expert(L[:, e], sel[:, e], M, mode, T, words[e])
        assert np.array_equal(got[:, e], exp_col), (e, L[:, e], sel[:, e], got[:, e], exp_col)
        c, c2 = int(sel[:, e].sum()), int(got[:, e].sum())
        assert c2 == target
        assert c2 % M == 0
        assert abs(c2 - c) < M
        if mode == 1 and c + (M - c % M) <= T:
            assert abs(c2 - c) <= M / 2


def test_token_rounding_weights_and_empty_tokens():
    rng = np.random.default_rng(5)
    T, E, K, M = 30, 6, 1, 8
    L = rng.normal(size=(T, E))
    plan = oracle.build_plan(L, K, round_mode=3, tile_m=M)     # DOWN: tokens can lose all experts
    assert np.all(plan["counts"] % M == 0)
    nk = plan["sel"].sum(axis=1)
    assert np.any(nk == 0)
    for t in range(T):
        s = plan["weights"][t].sum()
        assert (abs(s - 1.0) < 1e-15) if nk[t] else s == 0.0
    check_plan_identities(plan, T, E)


def test_kimi_scale_rounding_statistics():
    """NEAREST moves each count by at most half a tile; counts become tile multiples."""
    rng = np.random.default_rng(9)
    T, E, K, M = 4096, 48, 4, 128
    b = -1.1 * np.log(rng.permutation(E) + 1.0)
    L = rng.normal(size=(T, E)) * 0.5 + b
    plain = oracle.build_plan(L, K)
    tr = oracle.build_plan(L, K, round_mode=1, tile_m=M)
    assert np.all(tr["counts"] % M == 0)
    assert np.all(np.abs(tr["counts"] - plain["counts"]) <= M // 2)
    # rounding never touches a (token, expert) pair except at the boundary of its expert's ranking
    for e in range(E):
        order = np.lexsort((np.arange(T), -L[:, e]))
        m_plain = plain["sel"][order, e]
        m_tr = tr["sel"][order, e]
        changed = np.nonzero(m_plain != m_tr)[0]
        if len(changed):
            if tr["counts"][e] > plain["counts"][e]:
                assert not m_plain[changed].any()
                # every non-member ranked above an added token was added too
                first_left = np.nonzero(~m_tr)[0]
                assert len(first_left) == 0 or first_left.min() > changed.max()
            else:
                assert m_plain[changed].all()
                kept_after = np.nonzero(m_tr)[0]
                assert len(kept_after) == 0 or kept_after.max() < changed.min()


def test_stochastic_rounding_limits_and_threshold():
    """Word 0 rounds every partial expert up (as UP), the largest word rounds every one down (as
    DOWN); the switch sits exactly at word = ceil(r * 2^32 / M)."""
    rng = np.random.default_rng(21)
    T, E, K, M = 200, 12, 3, 16
    L = rng.normal(size=(T, E))
    up = oracle.build_plan(L, K, round_mode=2, tile_m=M)
    down = oracle.build_plan(L, K, round_mode=3, tile_m=M)
    zero = oracle.build_plan(L, K, round_mode=4, tile_m=M, round_rand=np.zeros(E, np.uint32))
    full = oracle.build_plan(L, K, round_mode=4, tile_m=M, round_rand=np.full(E, 2 ** 32 - 1, np.uint32))
    assert np.array_equal(zero["sel"], up["sel"]) and np.array_equal(full["sel"], down["sel"])
    plain = oracle.build_plan(L, K)
    for e in range(E):
        r = int(plain["counts"][e]) % M
        if r == 0:
            continue
        edge = -(-(r << 32) // M)          # smallest word that no longer rounds up
        words = np.zeros(E, np.uint32)
        for w, expect_up in ((edge - 1, True), (edge, False)):
            words[e] = w
            got = oracle.build_plan(L, K, round_mode=4, tile_m=M, round_rand=words)["counts"][e]
            assert got == (plain["counts"][e] - r + (M if expect_up else 0)), (e, r, w)


def test_stochastic_rounding_keeps_expected_counts():
    """Over independent words, each expert's mean rounded count matches its plain count (the
    SonicMoE page's claim that the expected total is kept): within 4 standard errors."""
    rng = np.random.default_rng(22)
    T, E, K, M = 300, 10, 2, 32
    L = rng.normal(size=(T, E))
    plain = oracle.build_plan(L, K)["counts"].astype(np.float64)
    n = 600
    acc = np.zeros(E)
    for _ in range(n):
        words = rng.integers(0, 2 ** 32, size=E, dtype=np.uint64).astype(np.uint32)
        acc += oracle.build_plan(L, K, round_mode=4, tile_m=M, round_rand=words)["counts"]
    mean = acc / n
    r = plain % M
    se = M * np.sqrt((r / M) * (1 - r / M) / n) + 1e-9
    assert np.all(np.abs(mean - plain) <= 4 * se + 1e-9), (mean, plain)

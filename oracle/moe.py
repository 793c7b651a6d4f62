"""Plain float64 definition of the one-GPU MoE layer (test infrastructure only).

Nothing here is blocked, fused or reordered: each function is the textbook statement of one step
of the layer, in the order the pages give the steps, with numpy matmuls as the only library
primitive.  Weight containers are only ever indexed as ``W[e]`` (one expert at a time), so a caller
may pass a lazy object that converts one expert's weights to float64 on demand; that is how the
largest layer shapes are checked without holding every expert in float64 at once.

Notation (the pages'): T tokens, d model width, n expert FFN width, E experts, K experts per
token, M the token-rounding tile.  ``L[T, E]`` are router logits, ``S_t`` the experts token t is
sent to, ``w_{t,e}`` its gate weights.  Rows of the permuted (expert-major) layout are indexed r.
"""

import numpy as np

ROUND_NONE, ROUND_NEAREST, ROUND_UP, ROUND_DOWN, ROUND_STOCHASTIC = 0, 1, 2, 3, 4


# ----------------------------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------------------------

def router_logits(X, W_r, bias=None):
    """Gate network: ``L = X W_r^T (+ b)``.

    cloud.baidu.com page, section "工作原理", step 1 of the pseudo-code (``router_logits =
    gate_network(tokens)``); apxml.com page, "自定义核与核融合", fused step 1 (gate scores).
    The per-expert bias ``b`` is an addition to the logits before both selection and weighting
    (the only place the workloads mention it is "router logits get a per-expert bias").
    """
    L = np.asarray(X, np.float64) @ np.asarray(W_r, np.float64).T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    return L


def topk_select(L, K):
    """Top-K selection: per token, the K experts with the largest logit.

    cloud.baidu.com page, "工作原理" (``expert_indices = top_k(router_logits)``); apxml.com page,
    fused step 2.  The pages do not say how ties are broken or in which order the K experts are
    listed.  Reading taken: the key order is (logit descending, expert id ascending), so a tie
    goes to the lower expert id, and the K ids are listed in that key order.  Selection uses the
    logits themselves: softmax is monotone, so selecting on probabilities picks the same set.
    """
    L = np.asarray(L, np.float64)
    # A stable sort of the negated keys lists equal keys in ascending expert id.
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :K].astype(np.int64)


def plain_topk_weights(L, topk_idx):
    """Softmax over each token's K selected logits (weights of plain top-K routing).

    The pages say only that outputs are combined "weighted by the gate scores" (apxml.com page,
    fused step 5).  Reading taken: the softmax taken over the selected experts, i.e. the full
    softmax renormalised over the selection, so that each token's weights sum to 1.
    """
    sel = np.take_along_axis(np.asarray(L, np.float64), topk_idx, axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


def _round_adds(c, M, mode, T, word=None):
    """Decide, for one expert with c tokens, whether token rounding adds or drops tokens.

    ``word`` is the expert's uniform 32-bit random word (stochastic mode only): with u = word / 2^32
    the expert rounds up iff u < r / M, i.e. with probability r / M, which keeps the expected count
    at c.  The comparison is done in integers (word * M < r * 2^32), so it is exact."""
    r = c % M
    if r == 0:
        return None, 0
    if mode == ROUND_NEAREST:
        add = 2 * r >= M          # exactly half a tile rounds up
    elif mode == ROUND_UP:
        add = True
    elif mode == ROUND_DOWN:
        add = False
    elif mode == ROUND_STOCHASTIC:
        add = int(word) * M < r * (1 << 32)
    else:
        raise ValueError("unknown rounding mode %r" % (mode,))
    if add and c + (M - r) > T:   # cannot add more tokens than exist: round down instead
        add = False
    return add, (M - r) if add else r


def token_rounding(L, sel, M, mode, round_rand=None):
    """Token rounding of per-expert token counts to multiples of the tile M.

    SonicMoE summary page, optimization 3 ("Token Rounding 路由算法"): each expert's token count
    is moved to a multiple of the tile size (128 in the page's example), never by more than one
    tile away from plain top-K, and the page claims the expected total is kept.

    The page's wording is contradictory (it says "round up", yet also that the expected total
    stays the same).  Reading taken, with UP and DOWN kept as explicit modes:

    * c = tokens the expert received from plain top-K, r = c mod M;
    * NEAREST: drop r tokens if r < M/2, otherwise add M - r (so half a tile rounds up);
      UP always adds M - r; DOWN always drops r; nothing changes when r = 0;
    * STOCHASTIC (the one reading under which the expected total is literally kept): add M - r
      with probability r / M, else drop r, decided by the caller's uniform 32-bit word
      ``round_rand[e]`` (see ``_round_adds``);
    * an addition that would need more than T tokens drops instead;
    * an expert ranks all T tokens by (L[t, e] descending, t ascending); it drops its r
      lowest-ranked members and adds its M - r highest-ranked non-members.

    ``sel`` is the boolean [T, E] membership of plain top-K; the rounded membership is returned.
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    out = np.array(sel, dtype=bool, copy=True)
    t_ids = np.arange(T)
    for e in range(E):
        member = out[:, e].copy()
        word = None if round_rand is None else int(np.uint32(round_rand[e]))
        add, amount = _round_adds(int(member.sum()), M, mode, T, word)
        if add is None:
            continue
        # Expert e's preference over tokens: larger logit first, then lower token id.
        rank_order = np.lexsort((t_ids, -L[:, e]))
        if add:
            cand = rank_order[~member[rank_order]]
            out[cand[:amount], e] = True
        else:
            cand = rank_order[member[rank_order]]
            out[cand[len(cand) - amount:], e] = False
    return out


def gate_weights(L, sel):
    """Gate weights over each token's final expert set.

    ``w_{t,e} = exp(L[t,e] - m_t) / sum_{e' in S_t} exp(L[t,e'] - m_t)`` for e in S_t and 0
    elsewhere, m_t the largest selected logit.  Without token rounding this equals
    ``plain_topk_weights``.  After token rounding the pages do not say how weights change;
    reading taken: renormalise over the final set (the weights of a token still sum to 1), and a
    token left with no expert has no weights and receives a zero output.
    """
    L = np.asarray(L, np.float64)
    W = np.zeros_like(L)
    for t in range(L.shape[0]):
        es = np.nonzero(sel[t])[0]
        if len(es) == 0:
            continue
        x = L[t, es]
        ex = np.exp(x - x.max())
        W[t, es] = ex / ex.sum()
    return W


def build_plan(L, K, round_mode=ROUND_NONE, tile_m=128, round_rand=None):
    """Routing plan: selection, optional token rounding, counts, offsets and permutation.

    Per-expert counts and their exclusive prefix sum give each expert one contiguous segment of
    rows in the permuted layout (the SonicMoE page's grouped GEMM reads "contiguous packed" or
    "gathered" inputs, section "Gather 与加载融合"; the ThunderEP article, section 2.2.2, moves
    rows by int32 index lists).  The pages fix no order inside a segment; reading taken: rows of
    an expert in ascending token id, and a token's rows listed in ascending expert id.

    Returns a dict of numpy arrays:
      topk_idx [T,K], topk_w [T,K]  plain top-K ids (descending key) and their softmax weights
      sel [T,E] bool                final membership (after token rounding if any)
      weights [T,E]                 final gate weights (0 outside sel)
      counts [E], expert_off [E+1]  rows per expert and their exclusive scan
      row_token [R], row_expert [R], row_w [R]   expert-major rows
      tok_off [T+1], tok_row [R]    token-major index of rows (CSR)
    """
    L = np.asarray(L, np.float64)
    T, E = L.shape
    topk_idx = topk_select(L, K)
    topk_w = plain_topk_weights(L, topk_idx)
    sel = np.zeros((T, E), dtype=bool)
    np.put_along_axis(sel, topk_idx, True, axis=1)
    if round_mode != ROUND_NONE:
        sel = token_rounding(L, sel, tile_m, round_mode, round_rand)
    weights = gate_weights(L, sel)

    counts = sel.sum(axis=0).astype(np.int64)
    expert_off = np.zeros(E + 1, np.int64)
    expert_off[1:] = np.cumsum(counts)
    row_token = np.concatenate([np.nonzero(sel[:, e])[0] for e in range(E)]).astype(np.int64) \
        if E else np.zeros(0, np.int64)
    row_expert = np.repeat(np.arange(E), counts).astype(np.int64)
    row_w = weights[row_token, row_expert]

    row_of = np.full((T, E), -1, np.int64)
    row_of[row_token, row_expert] = np.arange(len(row_token))
    tok_row = row_of[sel]                       # C order: token-major, experts ascending
    tok_off = np.zeros(T + 1, np.int64)
    tok_off[1:] = np.cumsum(sel.sum(axis=1))
    return dict(topk_idx=topk_idx, topk_w=topk_w, sel=sel, weights=weights, counts=counts,
                expert_off=expert_off, row_token=row_token, row_expert=row_expert, row_w=row_w,
                tok_off=tok_off, tok_row=tok_row)


# ----------------------------------------------------------------------------------------------
# Dispatch (local permutation) and combine
# ----------------------------------------------------------------------------------------------

def permute(X, row_token):
    """Gather token rows into expert-major order: ``X_perm[r] = X[row_token[r]]``.

    The single-GPU form of the dispatch step (cloud.baidu.com page, pseudo-code step 2): every
    expert is local, so dispatch is only a row gather.
    """
    return np.asarray(X)[np.asarray(row_token)]


def unpermute(X_perm, tok_row):
    """Inverse of ``permute`` on the token-major replicated layout: ``Z[i] = X_perm[tok_row[i]]``.

    Row i of Z is the i-th (token, expert) pair in token-major order, so ``unpermute(permute(X))``
    is X with each token repeated once per expert it was routed to.
    """
    return np.asarray(X_perm)[np.asarray(tok_row)]


def combine(Y_perm, tok_off, tok_row, row_w=None):
    """Gate-weighted combine: ``out[t] = sum_{r in rows(t)} w_r Y_perm[r]`` (ascending expert).

    apxml.com page, fused step 5 (combine the outputs weighted by the gate scores);
    cloud.baidu.com page, pseudo-code step 4 (results return to the token's position).
    ``row_w=None`` sums with unit weights (the transpose of ``permute``).
    """
    Y_perm = np.asarray(Y_perm, np.float64)
    T = len(tok_off) - 1
    out = np.zeros((T, Y_perm.shape[1]), np.float64)
    for t in range(T):
        for i in range(tok_off[t], tok_off[t + 1]):
            r = tok_row[i]
            out[t] += (1.0 if row_w is None else row_w[r]) * Y_perm[r]
    return out


# ----------------------------------------------------------------------------------------------
# Expert computation (forward)
# ----------------------------------------------------------------------------------------------

def _sigmoid(x):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def swiglu_expert_forward(Xe, Wg, Wu, Wd):
    """One SwiGLU expert on its rows: ``G = Xe Wg^T, U = Xe Wu^T, A = silu(G) U, Y = A Wd^T``.

    The SonicMoE page's kernel-comparison table fuses SwiGLU into the expert GEMM; the workloads
    name separate gate, up and down weights.  Reading taken: no biases, silu(g) = g sigmoid(g).
    Shapes: Xe [c, d], Wg and Wu [n, d], Wd [d, n].
    """
    Xe = np.asarray(Xe, np.float64)
    G = Xe @ np.asarray(Wg, np.float64).T
    U = Xe @ np.asarray(Wu, np.float64).T
    A = G * _sigmoid(G) * U
    Y = A @ np.asarray(Wd, np.float64).T
    return G, U, A, Y


def layer_forward(X, Wg, Wu, Wd, plan, experts=None):
    """Whole layer forward for a routing plan: local expert compute, then weighted combine.

    For each expert e (ascending): gather its rows, run the SwiGLU expert, and add
    ``w_r * Y_r`` into ``out[t_r]``.  ``experts`` restricts the work to a subset (then ``out``
    holds only that subset's contribution and H, A, Y_perm only its rows).
    Returns out [T, d], H [R, 2n] (= [G | U]), A [R, n] and Y_perm [R, d].
    """
    X = np.asarray(X, np.float64)
    T, d = X.shape
    off, row_token, row_w = plan["expert_off"], plan["row_token"], plan["row_w"]
    E = len(off) - 1
    R = int(off[-1])
    n = None
    out = np.zeros((T, d), np.float64)
    H = A = None
    Y_perm = np.zeros((R, d), np.float64)
    for e in (range(E) if experts is None else experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        toks = row_token[lo:hi]
        G, U, Ae, Y = swiglu_expert_forward(X[toks], Wg[e], Wu[e], Wd[e])
        if n is None:
            n = G.shape[1]
            H = np.zeros((R, 2 * n), np.float64)
            A = np.zeros((R, n), np.float64)
        H[lo:hi, :n], H[lo:hi, n:], A[lo:hi] = G, U, Ae
        Y_perm[lo:hi] = Y
        out[toks] += row_w[lo:hi, None] * Y      # a token occurs at most once per expert
    return dict(out=out, H=H, A=A, Y_perm=Y_perm)


def token_forward(X, Wg, Wu, Wd, plan, tokens):
    """``out[t]`` for selected tokens only, evaluating each of the token's experts on its row.

    Same arithmetic as ``layer_forward``, organised per token, for sampled checks of layer
    shapes whose full float64 evaluation is too large.
    """
    X = np.asarray(X, np.float64)
    res = np.zeros((len(tokens), X.shape[1]), np.float64)
    for j, t in enumerate(tokens):
        for i in range(plan["tok_off"][t], plan["tok_off"][t + 1]):
            r = plan["tok_row"][i]
            e = plan["row_expert"][r]
            _, _, _, Y = swiglu_expert_forward(X[t:t + 1], Wg[e], Wu[e], Wd[e])
            res[j] += plan["row_w"][r] * Y[0]
    return res


# ----------------------------------------------------------------------------------------------
# Backward
# ----------------------------------------------------------------------------------------------

def router_backward(dS, plan, T, E):
    """Gradient of the loss with respect to the logits through the gate weights.

    ``dS_r = dLoss/dw_r``.  For the softmax over the token's final set S_t:
    ``dL[t, j] = w_{t,j} (dS_{t,j} - sum_{k in S_t} w_{t,k} dS_{t,k})`` for j in S_t, 0 elsewhere.
    The discrete selection (top-K and token rounding) is held fixed, and the bias is a constant.
    """
    dL = np.zeros((T, E), np.float64)
    tok_off, tok_row = plan["tok_off"], plan["tok_row"]
    row_w, row_expert = plan["row_w"], plan["row_expert"]
    for t in range(T):
        rows = tok_row[tok_off[t]:tok_off[t + 1]]
        if len(rows) == 0:
            continue
        w = row_w[rows]
        s = np.dot(w, dS[rows])
        dL[t, row_expert[rows]] = w * (dS[rows] - s)
    return dL


def layer_backward(dY, X, Wg, Wu, Wd, plan, W_r=None, experts=None):
    """Backward of the layer for a fixed routing plan.

    SonicMoE page, optimization 1: nothing the router gradient needs is cached; the expert
    activations are recomputed from the inputs, which gives the same mathematics.  Here every
    activation is simply recomputed from X (the plainest form of that statement).  Section
    "反向传播优化" lists the gathers: dW1 (gate/up weights) reads gathered X, dW2 (down weight)
    and dH read gathered dO.  The router-score gradient uses ``dS_r = <dA'_r, A_r>`` with
    ``dA' = dY[t_r] Wd``, which equals ``<dY_t, Y_r>`` without forming Y (the page's
    "dS computation" row).

    For each expert e with rows r (tokens t_r, weights w_r):
      dA' = dY[t_r] Wd[e];  dS_r = <dA'_r, A_r>;  dA = w_r dA'
      dWd[e] = (w dY[t_r])^T A
      dG = dA * U * sigmoid(G) * (1 + G (1 - sigmoid(G)));  dU = dA * silu(G)
      dWg[e] = dG^T X[t_r];  dWu[e] = dU^T X[t_r];  dX[t_r] += dG Wg[e] + dU Wu[e]
    then dLogits by ``router_backward``; if ``W_r`` is given, also the router GEMM's backward:
    ``dX += dLogits W_r`` and ``dW_r = dLogits^T X``.

    ``experts`` restricts the expert loop to a subset (dX then holds only their share, and dS,
    dLogits, dW_r are only meaningful when every expert is included).
    """
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    T, d = X.shape
    off, row_token, row_w = plan["expert_off"], plan["row_token"], plan["row_w"]
    E = len(off) - 1
    R = int(off[-1])
    dX = np.zeros((T, d), np.float64)
    dS = np.zeros(R, np.float64)
    dWg, dWu, dWd = {}, {}, {}
    for e in (range(E) if experts is None else experts):
        lo, hi = int(off[e]), int(off[e + 1])
        Wg_e = np.asarray(Wg[e], np.float64)
        Wu_e = np.asarray(Wu[e], np.float64)
        Wd_e = np.asarray(Wd[e], np.float64)
        if hi == lo:
            dWg[e], dWu[e], dWd[e] = np.zeros_like(Wg_e), np.zeros_like(Wu_e), np.zeros_like(Wd_e)
            continue
        toks = row_token[lo:hi]
        w = row_w[lo:hi, None]
        Xe = X[toks]
        G, U, A, _ = swiglu_expert_forward(Xe, Wg_e, Wu_e, Wd_e)
        dYe = dY[toks]
        dA_raw = dYe @ Wd_e
        dS[lo:hi] = np.sum(dA_raw * A, axis=1)
        dA = w * dA_raw
        dWd[e] = (w * dYe).T @ A
        sg = _sigmoid(G)
        dG = dA * U * sg * (1.0 + G * (1.0 - sg))
        dU = dA * G * sg
        dWg[e] = dG.T @ Xe
        dWu[e] = dU.T @ Xe
        dX[toks] += dG @ Wg_e + dU @ Wu_e
    res = dict(dX=dX, dS=dS, dW_gate=dWg, dW_up=dWu, dW_down=dWd)
    if experts is None:
        dL = router_backward(dS, plan, T, E)
        res["dLogits"] = dL
        if W_r is not None:
            W_r = np.asarray(W_r, np.float64)
            res["dX_router"] = dL @ W_r
            res["dX"] = dX + res["dX_router"]
            res["dW_r"] = dL.T @ X
    return res

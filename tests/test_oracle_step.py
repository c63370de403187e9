"""Pins for the oracle's whole step and its per-head top-k (CPU only).

`step` is pinned on a tiny step whose every output is fixed by hand, not by
the oracle's own functions: W1 = 0 (so r = h exactly) and W2_k a cyclic
shift, so each head's logits, top-k and the tree's tokens are known in
closed form; equal keys everywhere, so tree attention is the mean of the
values a node may see; one-hot-like verification rows, so the accepted path
is chosen by hand.  A stage dropped, swapped or fed the wrong input changes
one of these outputs.  `topk_per_head` is pinned against a full sort of each
head's rows (Python's sorted on (-value, index)).
"""
import math

import numpy as np
import pytest

import oracle


def test_topk_per_head_brute_force():
    g = np.random.default_rng(0)
    K, M, V, k = 3, 4, 50, 6
    x = np.round(g.standard_normal((K, M, V)) * 2) / 2     # coarse grid: many ties
    x[1, 2, :] = 0.0                                        # one row of all-equal values
    x[2, 0, 7] = -0.0
    idx, val = oracle.topk_per_head(x, k)
    assert idx.shape == (K, M, k) and val.shape == (K, M, k)
    for h in range(K):
        for m in range(M):
            order = sorted(range(V), key=lambda v: (-x[h, m, v], v))[:k]
            assert idx[h, m].tolist() == order, (h, m)
            assert val[h, m].tolist() == [x[h, m, v] for v in order]
    assert idx[1, 2].tolist() == list(range(k))            # all equal: lowest ids first
    # rows and heads stay apart: a row's answer depends on that row alone
    y = x.copy()
    y[0, 1] = y[0, 1][::-1]
    idx2, _ = oracle.topk_per_head(y, k)
    assert np.array_equal(np.delete(idx2.reshape(K * M, k), 1, axis=0), np.delete(idx.reshape(K * M, k), 1, axis=0))
    assert idx2[0, 1].tolist() == sorted(range(V), key=lambda v: (-y[0, 1, v], v))[:k]


# paths of the hand-worked tree (K = 3 heads, top-2 each): node order is
# root, then by (length, lexicographic)
PATHS = [[0], [1], [0, 0], [0, 1], [1, 0], [0, 0, 0]]
#         1    2     3       4       5        6
PARENT = [-1, 0, 0, 1, 1, 2, 3]
DEPTH = [0, 1, 1, 2, 2, 2, 3]
RANK = [-1, 0, 1, 0, 1, 0, 0]


def hand_step(B=2, V=8, nh=2, dh=4, L=3, eps=0.09, delta=0.3, hot=30.0):
    """Inputs and expected outputs of the tiny step, written out by hand."""
    H, K, k, T = V, 3, 2, 7
    # h[b][i] = (V - i) + 10 b: strictly decreasing in i, small integers (exact in bf16)
    h = np.array([[float(V - i + 10 * b) for i in range(H)] for b in range(B)])
    W1 = np.zeros((K, H, H))
    # W2_k[v][i] = 1 iff i = (v + k) mod V, so logits_k[b][v] = h[b][(v + k) mod V]
    W2 = np.zeros((K, V, H))
    for kk in range(K):
        for v in range(V):
            W2[kk, v, (v + kk) % V] = 1.0
    exp_logits = np.array([[[h[b][(v + kk) % V] for v in range(V)] for b in range(B)] for kk in range(K)])
    # largest h[b][i] is at i = 0, then 1, ...: head k's rank-r token v has (v + k) mod V = r
    exp_idx = np.array([[[(r - kk) % V for r in range(k)] for b in range(B)] for kk in range(K)])
    root = np.array([5, 2][:B])
    exp_tok = np.array([[root[b]] + [(RANK[j] - (DEPTH[j] - 1)) % V for j in range(1, T)] for b in range(B)])
    # attention: every key equal (scores equal), value rows distinct; node j sees the L
    # cache rows and its ancestors incl. itself, so o_j = their plain mean
    q = np.ones((B, T, nh, dh))
    kt = np.ones((B, T, nh, dh))
    kc = np.ones((B, nh, L, dh))
    vt = np.array([[[[100.0 * j + 10 * hh + d + b for d in range(dh)] for hh in range(nh)] for j in range(T)]
                   for b in range(B)])
    vc = np.array([[[[-(1.0 + c) * (hh + 1) + d * b for d in range(dh)] for c in range(L)] for hh in range(nh)]
                   for b in range(B)])
    anc = {0: [0], 1: [0, 1], 2: [0, 2], 3: [0, 1, 3], 4: [0, 1, 4], 5: [0, 2, 5], 6: [0, 1, 3, 6]}
    exp_attn = np.empty((B, T, nh, dh))
    for b in range(B):
        for j in range(T):
            for hh in range(nh):
                rows = [vc[b, hh, c] for c in range(L)] + [vt[b, a, hh] for a in anc[j]]
                exp_attn[b, j, hh] = sum(rows) / len(rows)
    # verification rows: row n puts 30 on one chosen token, 0 elsewhere.  The chosen
    # token of the root row is node 2's token for sequence 0 (so (1) is accepted,
    # (0) is not), node 1's for sequence 1; deeper rows pick the child to follow.
    target = {0: {0: 2, 2: 5, 5: None}, 1: {0: 1, 1: 3, 3: 6, 6: None}}
    vl = np.zeros((B, T, V))
    for b in range(B):
        for n in range(T):
            child = target[b].get(n)
            t_tok = exp_tok[b, child] if child is not None else (n + 3 * b) % V
            vl[b, n, t_tok] = hot
    # p(target) = e^hot / (e^hot + V - 1), every other token 1 / (e^hot + V - 1):
    # above and below thr = min(eps, delta e^-H) for the (hot, eps, delta) used
    # here, so the accepted path is the target chain
    exp_best = {0: 5, 1: 6}
    exp_len = {0: 2, 1: 3}
    exp_path = {0: [0, 2, 5], 1: [0, 1, 3, 6]}
    exp_next = {b: (exp_best[b] + 3 * b) % V for b in range(B)}
    tree = oracle.build_tree(PATHS, K, k)
    return dict(h=h, W1=W1, W2=W2, root=root, tree=tree, k=k, q=q, kt=kt, vt=vt, kc=kc, vc=vc, vl=vl, eps=eps,
                delta=delta, exp_logits=exp_logits, exp_idx=exp_idx, exp_tok=exp_tok, exp_attn=exp_attn,
                exp_best=exp_best, exp_len=exp_len, exp_path=exp_path, exp_next=exp_next)


def check_step(out, c, B):
    tree = c["tree"]
    assert tree["parent"].tolist() == PARENT and tree["depth"].tolist() == DEPTH and tree["rank"].tolist() == RANK
    assert np.array_equal(out["head_logits"], c["exp_logits"])
    assert np.array_equal(out["topk_idx"], c["exp_idx"])
    assert np.array_equal(out["tree_tok"], c["exp_tok"])
    assert np.allclose(out["attn"], c["exp_attn"], rtol=0, atol=1e-9)
    acc = out["accept"]
    for b in range(B):
        assert acc["best"][b] == c["exp_best"][b]
        assert acc["accept_len"][b] == c["exp_len"][b]
        path_tok = [c["exp_tok"][b, j] for j in c["exp_path"][b]]
        assert acc["accepted_tok"][b, :len(path_tok)].tolist() == path_tok
        assert (acc["accepted_tok"][b, len(path_tok):] == -1).all()
        assert acc["next_tok"][b] == c["exp_next"][b]


@pytest.mark.parametrize("round_r,hot,eps", [(False, 30.0, 0.09), (True, 30.0, 0.09), (False, 3.0, 0.2)])
def test_step_hand_worked(round_r, hot, eps):
    # hot = 3: p(target) = 0.741, others 0.037, H = 1.07 nats: thr = delta e^-H = 0.1025
    # (below eps = 0.2), so eps and delta swapped would give 0.068 instead
    B = 2
    c = hand_step(B, hot=hot, eps=eps)
    out = oracle.step(c["h"], c["W1"], c["W2"], c["root"], c["tree"], c["k"], c["q"], c["kt"], c["vt"], c["kc"],
                      c["vc"], c["vl"], c["eps"], c["delta"], temperature=1.0, round_r_bf16=round_r)
    check_step(out, c, B)
    # the thresholds are the closed form min(eps, delta e^-H) of the planted rows
    V = c["vl"].shape[2]
    Z = math.exp(hot) + V - 1
    p_hi, p_lo = math.exp(hot) / Z, 1.0 / Z
    H = -(p_hi * math.log(p_hi) + (V - 1) * p_lo * math.log(p_lo))
    thr = min(c["eps"], c["delta"] * math.exp(-H))
    assert np.isclose(out["accept"]["thr"][0, 1], thr, rtol=1e-12)
    assert np.isclose(out["accept"]["p"][0, 2], p_hi, rtol=1e-12)
    assert np.isclose(out["accept"]["p"][0, 1], p_lo, rtol=1e-12)
    if hot == 3.0:
        assert 0.102 < thr < 0.103 and p_lo < thr < p_hi


def test_step_verification_logits_from_the_candidates():
    # the verification logits may be a function of the step's own candidate tokens:
    # it must see exactly the tree tokens the heads produced
    B = 2
    c = hand_step(B)
    seen = []

    def vfn(tok):
        seen.append(np.array(tok))
        return c["vl"]

    out = oracle.step(c["h"], c["W1"], c["W2"], c["root"], c["tree"], c["k"], c["q"], c["kt"], c["vt"], c["kc"],
                      c["vc"], vfn, c["eps"], c["delta"])
    assert len(seen) == 1 and np.array_equal(seen[0], c["exp_tok"])
    check_step(out, c, B)


def test_step_temperature_zero_is_greedy_walk():
    # temperature 0: each row is one-hot at its argmax, so the accepted path
    # follows the argmax tokens: the same hand-worked answer
    # (rows of moderate entropy, where temperature 1 would give thr = 0.1025): at
    # temperature 0, p is exactly 1 or 0 and thr = min(eps, delta) = 0.2
    B = 2
    c = hand_step(B, hot=3.0, eps=0.2)
    out = oracle.step(c["h"], c["W1"], c["W2"], c["root"], c["tree"], c["k"], c["q"], c["kt"], c["vt"], c["kc"],
                      c["vc"], c["vl"], c["eps"], c["delta"], temperature=0.0)
    check_step(out, c, B)
    assert np.all(out["accept"]["thr"][:, 1:] == 0.2)
    assert set(np.unique(out["accept"]["p"][:, 1:]).tolist()) == {0.0, 1.0}

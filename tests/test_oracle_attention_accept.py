"""Pins for the oracle's tree attention and typical acceptance (CPU only)."""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax
from scipy.stats import entropy

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def inputs(B, T, nh, dh, L, seed=0):
    q = rnd((B, T, nh, dh), seed)
    kt = rnd((B, T, nh, dh), seed + 1)
    vt = rnd((B, T, nh, dh), seed + 2)
    kc = rnd((B, nh, L, dh), seed + 3)
    vc = rnd((B, nh, L, dh), seed + 4)
    return q, kt, vt, kc, vc


# ---------------------------------------------------------------- attention
def test_chain_tree_equals_token_by_token_causal_decode():
    # a chain tree is ordinary causal attention: decode token j after
    # appending tokens 0..j to the cache
    B, nh, dh, L, D = 2, 3, 16, 9, 5
    tree = oracle.build_tree([[0] * d for d in range(1, D + 1)], D, 1)
    q, kt, vt, kc, vc = inputs(B, D + 1, nh, dh, L, seed=10)
    got = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    for b in range(B):
        for h in range(nh):
            Kc, Vc = list(kc[b, h]), list(vc[b, h])
            for j in range(D + 1):
                Kc.append(kt[b, j, h])
                Vc.append(vt[b, j, h])
                w = softmax(np.array(Kc) @ q[b, j, h] / math.sqrt(dh))
                assert np.allclose(got[b, j, h], w @ np.array(Vc), rtol=1e-12, atol=1e-12)


def test_single_node_is_plain_decode_attention():
    B, nh, dh, L = 1, 2, 8, 30
    tree = oracle.build_tree([[0]], 1, 1)
    q, kt, vt, kc, vc = inputs(B, 2, nh, dh, L, seed=20)
    got = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    for h in range(nh):
        keys = np.vstack([kc[0, h], kt[0, 0, h]])
        vals = np.vstack([vc[0, h], vt[0, 0, h]])
        ref = softmax(keys @ q[0, 0, h] / math.sqrt(dh)) @ vals
        assert np.allclose(got[0, 0, h], ref, rtol=1e-12, atol=1e-12)


def test_equal_keys_average_exactly_the_visible_values():
    # identical keys -> uniform weights over prefix + ancestors (+ self)
    B, nh, dh, L = 1, 1, 4, 6
    tree = oracle.build_tree(oracle.dense_paths(3, 2), 3, 2)
    T = tree["T"]
    q, _, vt, _, vc = inputs(B, T, nh, dh, L, seed=30)
    kt = np.ones((B, T, nh, dh))
    kc = np.ones((B, nh, L, dh))
    got = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    for j in range(T):
        chain = []
        i = j
        while i != -1:
            chain.append(i)
            i = tree["parent"][i]
        vis = np.vstack([vc[0, 0], vt[0, chain, 0]])
        assert len(vis) == L + tree["depth"][j] + 1
        assert np.allclose(got[0, j, 0], vis.mean(axis=0), rtol=1e-12, atol=1e-12)


def test_constant_values_and_empty_prefix():
    B, nh, dh, L = 2, 2, 8, 0
    tree = oracle.build_tree(oracle.dense_paths(2, 3), 2, 3)
    q, kt, _, kc, _ = inputs(B, tree["T"], nh, dh, L, seed=40)
    v = rnd((dh,), 41)
    vt = np.broadcast_to(v, (B, tree["T"], nh, dh)).copy()
    vc = np.zeros((B, nh, 0, dh))
    got = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    assert np.allclose(got, np.broadcast_to(v, got.shape), rtol=1e-12, atol=1e-12)


def test_non_ancestors_do_not_leak_and_prefix_order_is_irrelevant():
    B, nh, dh, L = 1, 2, 8, 12
    tree = oracle.build_tree(oracle.dense_paths(3, 2), 3, 2)
    T = tree["T"]
    q, kt, vt, kc, vc = inputs(B, T, nh, dh, L, seed=50)
    base = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    j = T - 1
    anc = set(oracle.ancestors(tree, j))
    kt2, vt2 = kt.copy(), vt.copy()
    for i in range(T):
        if i not in anc:
            kt2[:, i] += 5.0
            vt2[:, i] -= 3.0
    pert = oracle.tree_attention(q, kt2, vt2, kc, vc, tree)
    assert np.array_equal(pert[:, j], base[:, j])
    perm = np.random.default_rng(51).permutation(L)
    shuf = oracle.tree_attention(q, kt, vt, kc[:, :, perm], vc[:, :, perm], tree)
    assert np.allclose(shuf, base, rtol=1e-12, atol=1e-12)


def test_default_scale_closed_form():
    # prefix keys 0 and a*e0, root key 0, query c*e0:
    # weights proportional to (1, exp(a c / sqrt(dh)), 1)
    dh, a, c = 16, 1.5, 2.0
    tree = oracle.build_tree([], 1, 1)          # the root alone
    q = np.zeros((1, 1, 1, dh)); q[0, 0, 0, 0] = c
    kc = np.zeros((1, 1, 2, dh)); kc[0, 0, 1, 0] = a
    vc = np.zeros((1, 1, 2, dh)); vc[0, 0, 0, 1] = 1.0; vc[0, 0, 1, 2] = 1.0
    kt = np.zeros((1, 1, 1, dh)); vt = np.zeros((1, 1, 1, dh)); vt[0, 0, 0, 3] = 1.0
    o = oracle.tree_attention(q, kt, vt, kc, vc, tree)[0, 0, 0]
    e = math.exp(a * c / 4.0)
    assert np.allclose(o[1:4], [1 / (2 + e), e / (2 + e), 1 / (2 + e)], rtol=1e-14)


# ---------------------------------------------------------------- acceptance
def tree_and_tokens(K, k, B, V, seed):
    tree = oracle.build_tree(oracle.dense_paths(K, k), K, k)
    g = np.random.default_rng(seed)
    idx = np.stack([np.stack([g.choice(V, k, replace=False) for _ in range(B)]) for _ in range(K)])
    tok = oracle.tree_tokens(tree, g.integers(0, V, B), idx)
    return tree, tok


def greedy_walk(logits_b, tok_b, tree):
    """Greedy verification written as a walk down the tree."""
    n = 0
    while True:
        am = int(np.argmax(logits_b[n]))
        nxt = [c for c in range(1, tree["T"]) if tree["parent"][c] == n and tok_b[c] == am]
        if not nxt:
            return int(tree["depth"][n]), n, am
        n = min(nxt)


@pytest.mark.parametrize("seed", range(4))
def test_temperature_zero_is_greedy_verification(seed):
    B, V = 3, 12
    tree, tok = tree_and_tokens(3, 3, B, V, seed)
    g = np.random.default_rng(100 + seed)
    logits = g.standard_normal((B, tree["T"], V))
    # plant argmaxes on candidate tokens so that greedy walks go deep
    for b in range(B):
        for n in range(tree["T"]):
            kids = [c for c in range(1, tree["T"]) if tree["parent"][c] == n]
            if kids and g.random() < 0.7:
                logits[b, n, tok[b, kids[g.integers(len(kids))]]] += 10
    res = oracle.typical_accept(logits, tok, tree, 0.09, 0.3, temperature=0.0)
    for b in range(B):
        alen, best, nxt = greedy_walk(logits[b], tok[b], tree)
        assert res["accept_len"][b] == alen
        assert res["best"][b] == best
        assert res["next_tok"][b] == nxt


def test_eps_to_zero_accepts_everything():
    B, V = 2, 20
    tree, tok = tree_and_tokens(3, 2, B, V, 7)
    logits = np.clip(np.random.default_rng(8).standard_normal((B, tree["T"], V)) * 3, -10, 10)
    res = oracle.typical_accept(logits, tok, tree, 1e-300, 0.3, 1.0)
    deepest = int(np.flatnonzero(tree["depth"] == tree["depth_max"])[0])
    assert (res["accept_len"] == tree["depth_max"]).all()
    assert (res["best"] == deepest).all()


def test_delta_large_is_fixed_posterior_threshold():
    # delta -> inf: threshold = eps, the fixed-threshold rule (with '>')
    B, V, eps = 2, 16, 0.09
    tree, tok = tree_and_tokens(2, 3, B, V, 9)
    logits = np.random.default_rng(10).standard_normal((B, tree["T"], V)) * 2
    res = oracle.typical_accept(logits, tok, tree, eps, 1e300, 1.0)
    for b in range(B):
        for c in range(1, tree["T"]):
            p = softmax(logits[b, tree["parent"][c]])[tok[b, c]]
            assert res["dec"][b, c] == (p > eps)


def test_entropy_threshold_against_scipy():
    B, V, eps, delta = 2, 40, 0.09, 0.3
    tree, tok = tree_and_tokens(2, 2, B, V, 11)
    logits = np.random.default_rng(12).standard_normal((B, tree["T"], V)) * 2.5
    for tau in (1.0, 0.7, 1.6):
        res = oracle.typical_accept(logits, tok, tree, eps, delta, tau)
        for b in range(B):
            for c in range(1, tree["T"]):
                P = softmax(logits[b, tree["parent"][c]] / tau)
                thr = min(eps, delta * math.exp(-entropy(P)))
                assert math.isclose(res["thr"][b, c], thr, rel_tol=1e-12)
                assert math.isclose(res["p"][b, c], P[tok[b, c]], rel_tol=1e-12)


def test_one_hot_and_uniform_rows():
    V = 50
    tree = oracle.build_tree([[0], [1]], 1, 2)
    tok = np.array([[3, 4, 5]])
    onehot = np.full((1, 3, V), -np.inf)
    onehot[0, :, 4] = 0.0
    P, H, am = oracle.row_distribution(onehot[0, 0], 1.0)
    assert H == 0.0 and am == 4
    res = oracle.typical_accept(onehot, tok, tree, 0.5, 0.3, 1.0)
    assert res["thr"][0, 1] == 0.3 and res["dec"][0].tolist() == [False, True, False]
    uni = np.zeros((1, 3, V))
    P, H, am = oracle.row_distribution(uni[0, 0], 1.0)
    assert math.isclose(H, math.log(V), rel_tol=1e-14) and am == 0
    # p = 1/V > delta/V for delta < 1: every candidate is accepted whatever eps
    res = oracle.typical_accept(uni, tok, tree, 0.9, 0.3, 1.0)
    assert res["dec"][0, 1:].all() and res["accept_len"][0] == 1 and res["best"][0] == 1


def test_strict_inequality():
    tree = oracle.build_tree([[0]], 1, 1)
    tok = np.array([[0, 1]])
    logits = np.zeros((1, 2, 2))                 # p = 0.5 each
    assert oracle.typical_accept(logits, tok, tree, 0.5, 1e300, 1.0)["accept_len"][0] == 0
    assert oracle.typical_accept(logits, tok, tree, 0.4999, 1e300, 1.0)["accept_len"][0] == 1


@pytest.mark.parametrize("seed", range(5))
def test_scan_equals_brute_force_over_paths(seed):
    B, V = 3, 10
    tree, tok = tree_and_tokens(3, 3, B, V, 200 + seed)
    logits = np.random.default_rng(300 + seed).standard_normal((B, tree["T"], V)) * 1.5
    res = oracle.typical_accept(logits, tok, tree, 0.2, 0.6, 1.0)
    for b in range(B):
        dec = res["dec"][b]
        ok = []
        for c in range(tree["T"]):
            chain = oracle.ancestors(tree, c)
            if all(dec[i] for i in chain if i != 0):
                ok.append(c)
        alen = max(int(tree["depth"][c]) for c in ok)
        best = min(c for c in ok if tree["depth"][c] == alen)
        assert res["accept_len"][b] == alen and res["best"][b] == best
        chain = oracle.ancestors(tree, best)
        assert res["accepted_tok"][b, :len(chain)].tolist() == tok[b, chain].tolist()
        assert (res["accepted_tok"][b, len(chain):] == -1).all()
        assert res["next_tok"][b] == int(np.argmax(logits[b, best]))


def test_peaked_scores_do_not_overflow():
    # scores in the thousands: the weight collapses onto the best key
    B, nh, dh, L = 1, 1, 8, 5
    tree = oracle.build_tree([[0]], 1, 1)
    q, kt, vt, kc, vc = inputs(B, 2, nh, dh, L, seed=60)
    q *= 2000.0
    got = oracle.tree_attention(q, kt, vt, kc, vc, tree)
    for j, chain in ((0, [0]), (1, [0, 1])):
        keys = np.vstack([kc[0, 0], kt[0, chain, 0]])
        vals = np.vstack([vc[0, 0], vt[0, chain, 0]])
        assert np.isfinite(got[0, j, 0]).all()
        assert np.allclose(got[0, j, 0], vals[np.argmax(keys @ q[0, j, 0])], atol=1e-12)

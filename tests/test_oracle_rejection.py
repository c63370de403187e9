"""Pins for the oracle's rejection-sampling acceptance (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle


def dists(V, seed):
    g = np.random.default_rng(seed)
    return g.dirichlet(np.ones(V)), g.dirichlet(np.ones(V) * 0.5)


@pytest.mark.parametrize("seed", range(4))
def test_one_draft_preserves_the_target_distribution(seed):
    # draft x ~ q, keep with min(1, p/q), else sample the residual: the
    # emitted token is distributed exactly as p (speculative sampling)
    p, q = dists(6, seed)
    out = np.zeros_like(p)
    res = oracle.rs_residual(p, q)
    for x in range(len(p)):
        a = oracle.rs_accept_prob(p, q, x)
        out[x] += q[x] * a
        out += q[x] * (1 - a) * res
    assert np.allclose(out, p, rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed", range(3))
def test_three_sibling_drafts_preserve_the_target_distribution(seed):
    # siblings drafted i.i.d. from q and tried in turn against the residual
    # of the rejected ones: still exactly p
    p, q = dists(4, 10 + seed)
    out = np.zeros_like(p)
    for xs in itertools.product(range(len(p)), repeat=3):
        w = np.prod(q[list(xs)])
        cur, alive = p, 1.0
        for x in xs:
            a = oracle.rs_accept_prob(cur, q, x)
            out[x] += w * alive * a
            alive *= 1 - a
            cur = oracle.rs_residual(cur, q)
        out += w * alive * cur
    assert np.allclose(out, p, rtol=0, atol=1e-13)


def test_sample_inverse_cdf_against_searchsorted():
    g = np.random.default_rng(3)
    p = g.random(50)
    p[[0, 7, 8, 49]] = 0.0
    for u in list(g.random(200)) + [0.0]:
        v = oracle.sample_inverse_cdf(p, u)
        c = np.cumsum(p)
        assert v == int(np.searchsorted(c, u * c[-1], side="right"))
        assert p[v] > 0


def random_case(T_paths, K, k, B, V, seed):
    tree = oracle.build_tree(T_paths, K, k)
    g = np.random.default_rng(seed)
    logits = g.standard_normal((B, tree["T"], V)) * 3
    head = g.standard_normal((K, B, V)) * 3
    tok = g.integers(0, V, (B, tree["T"]))
    return tree, logits, head, tok, g


@pytest.mark.parametrize("seed", range(5))
def test_temperature_zero_is_greedy_verification(seed):
    # one-hot p and q: a child is kept iff its token is the argmax of its
    # parent's row, whatever the uniforms -- typical acceptance at
    # temperature 0 takes the same decisions
    tree, logits, head, tok, g = random_case(oracle.dense_paths(3, 3), 3, 3, 4, 6, seed)
    # make some candidates the argmax so that paths get accepted
    for b in range(4):
        for c in range(1, tree["T"]):
            if g.random() < 0.5:
                tok[b, c] = int(np.argmax(logits[b, tree["parent"][c]]))
    r = oracle.rejection_accept(logits, head, tok, tree, 0.0, g.random((4, tree["T"])), g.random(4))
    t = oracle.typical_accept(logits, tok, tree, 0.09, 0.3, 0.0)
    for key in ("accept_len", "best", "next_tok", "accepted_tok"):
        assert np.array_equal(r[key], t[key]), key


def test_uniform_extremes_walk_the_tree():
    # chain tree: uniforms 0 keep every drafted token with p(x) > 0 (all, at
    # temperature 1), so the walk reaches the leaf and samples from its row;
    # uniforms just below 1 keep only tokens with p(x) >= q(x)
    D, V, B = 4, 8, 3
    tree, logits, head, tok, g = random_case([[0] * d for d in range(1, D + 1)], D, 1, B, V, 7)
    r = oracle.rejection_accept(logits, head, tok, tree, 1.0, np.zeros((B, D + 1)), np.full(B, 0.5))
    assert r["accept_len"].tolist() == [D] * B and r["best"].tolist() == [D] * B
    for b in range(B):
        P, _, _ = oracle.row_distribution(logits[b, D], 1.0)
        assert r["next_tok"][b] == oracle.sample_inverse_cdf(P, 0.5)
    hi = np.nextafter(1.0, 0.0)
    r = oracle.rejection_accept(logits, head, tok, tree, 1.0, np.full((B, D + 1), hi), np.full(B, 0.25))
    for b in range(B):
        u, n = 0, 0
        while n < D:
            p, _, _ = oracle.row_distribution(logits[b, u], 1.0)
            q, _, _ = oracle.row_distribution(head[u, b], 1.0)
            x = tok[b, u + 1]
            if not p[x] >= q[x]:
                break
            u, n = u + 1, n + 1
        assert r["accept_len"][b] == n


def test_rejected_siblings_use_the_residual():
    # root with three children, the first two rejected (uniform ~1, their
    # tokens have p < q), the third tested against the twice-updated residual
    tree = oracle.build_tree([[0], [1], [2]], 1, 3)
    V = 5
    z = np.log(np.array([[0.05, 0.05, 0.4, 0.3, 0.2]]))
    qz = np.log(np.array([[0.5, 0.3, 0.1, 0.05, 0.05]]))
    logits = np.repeat(z[:, None, :], 4, axis=1)
    head = qz[None]
    tok = np.array([[0, 0, 1, 3]])
    hi = np.nextafter(1.0, 0.0)
    u = np.array([[0.0, hi, hi, 0.7]])
    r = oracle.rejection_accept(logits, head, tok, tree, 1.0, u, np.array([0.5]))
    p, q = np.exp(z[0]), np.exp(qz[0])
    p1 = oracle.rs_residual(p, q)
    p2 = oracle.rs_residual(p1, q)
    assert r["a"][0, 1] == pytest.approx(0.1) and r["a"][0, 2] == pytest.approx(p1[1] / 0.3)
    a3 = min(1.0, p2[3] / q[3])
    assert r["a"][0, 3] == pytest.approx(a3)
    assert r["best"][0] == (3 if 0.7 < a3 else 0)

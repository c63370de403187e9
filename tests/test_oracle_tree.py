"""Pins for the oracle's candidate-tree functions (CPU only).

Each check is against something other than the oracle's own formula:
trees printed on the pages (tests/golden/page_trees.json), closed-form
counts, brute-force enumeration, and parent-chain walks.
"""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from speculative_decoding_05_amd import configs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_trees.json")))


def mask_sets(tree):
    out = []
    for j in range(tree["T"]):
        s = []
        for i in range(tree["T"]):
            if (int(tree["mask"][j, i // 64]) >> (i % 64)) & 1:
                s.append(i)
        out.append(s)
    return out


@pytest.mark.parametrize("name", ["two_heads_top2", "choices_standard", "choices_aggressive"])
def test_page_trees(name):
    g = GOLD[name]
    t = oracle.build_tree(g["paths"], g["K"], g["k"])
    assert t["T"] == g["T"]
    assert t["n_leaves"] == g["n_leaves"]
    assert t["parent"].tolist() == g["parent"]
    assert mask_sets(t) == g["ancestors"]


@pytest.mark.parametrize("case", GOLD["dense_leaf_counts"])
def test_dense_leaf_counts_from_page(case):
    t = oracle.build_tree(oracle.dense_paths(case["K"], case["k"]), case["K"], case["k"])
    assert t["n_leaves"] == case["leaves"]
    # closed form: sum_{d=1..K} k^d non-root nodes
    assert t["T"] - 1 == sum(case["k"] ** d for d in range(1, case["K"] + 1))


def test_dense_config_sizes():
    assert oracle.build_tree(oracle.dense_paths(2, 2), 2, 2)["T"] == 7
    t = oracle.build_tree(oracle.dense_paths(4, 4), 4, 4)
    assert t["T"] == 341 and t["n_leaves"] == 256 and t["W"] == 6
    assert sum(int(t["depth"][j]) + 1 for j in range(t["T"])) == 1593


def test_leaf_count_is_product_rule():
    # Cartesian product of K top-k lists: k^K full-length candidates
    for K, k in [(1, 5), (2, 3), (3, 2), (3, 3)]:
        t = oracle.build_tree(oracle.dense_paths(K, k), K, k)
        full = list(itertools.product(range(k), repeat=K))
        leaves = [tuple(t["paths"][j - 1]) for j in range(1, t["T"]) if j not in set(t["parent"][1:])]
        assert sorted(leaves) == sorted(full)


def brute_greedy(K, rank_cap, n):
    """Rank every path by exact score (ties: shorter, then lexicographic)."""
    allp = []
    for d in range(1, K + 1):
        for p in itertools.product(range(rank_cap), repeat=d):
            s = Fraction(1)
            for hd, i in enumerate(p):
                s *= configs.acc_exact(hd, i)
            allp.append((-s, d, p))
    allp.sort()
    return allp


def test_greedy_tree_is_top_by_score_and_closed_form():
    ranked = brute_greedy(4, 10, 63)
    assert len(ranked) == 11110
    top = [p for _, _, p in ranked[:63]]
    got = oracle.greedy_paths(configs.acc_exact, 4, 63, 10)
    assert sorted(got) == sorted(top)
    # unique cut: the 63rd and 64th scores differ, with all ties inside / outside
    s63, s64 = -ranked[62][0], -ranked[63][0]
    assert s63 == Fraction(3, 5) ** 4 * Fraction(4, 5) ** 6 * Fraction(1, 2) ** 2
    assert s64 == Fraction(3, 5) ** 3 * Fraction(4, 5) ** 3 * Fraction(1, 2) ** 4
    # closed form: depth-d paths with rank sum <= (6, 5, 3, 2)
    cap = {1: 6, 2: 5, 3: 3, 4: 2}
    closed = [p for d in range(1, 5) for p in itertools.product(range(10), repeat=d) if sum(p) <= cap[d]]
    assert sorted(closed) == sorted(got)
    t = oracle.build_tree(got, 4, 10)
    assert t["T"] == 64 and t["n_leaves"] == 37 and t["depth_max"] == 4
    assert sum(int(t["depth"][j]) + 1 for j in range(t["T"])) == 233
    # five heads: the fifth head is never used by the 63 best paths
    assert sorted(oracle.greedy_paths(configs.acc_exact, 5, 63, 10)) == sorted(got)


def test_greedy_adds_frontier_nodes_only():
    got = oracle.greedy_paths(configs.acc_exact, 4, 63, 10)
    seen = set()
    for p in got:
        assert len(p) == 1 or p[:-1] in seen
        seen.add(p)


@pytest.mark.parametrize("paths,K,k", [
    ([[0, 0]], 2, 2),                 # prefix [0] missing
    ([[0], [0]], 2, 2),               # duplicate
    ([[2]], 2, 2),                    # rank >= k
    ([[0], [0, 0], [0, 0, 0]], 2, 2),  # depth > K
    ([[]], 2, 2),                     # empty path
    ([[-1]], 2, 2),                   # negative rank
])
def test_invalid_trees_rejected(paths, K, k):
    with pytest.raises(oracle.TreeError):
        oracle.build_tree(paths, K, k)


@st.composite
def prefix_closed_trees(draw):
    K = draw(st.integers(1, 5))
    k = draw(st.integers(1, 6))
    n = draw(st.integers(1, 120))
    paths = set()
    frontier = [(i,) for i in range(k)]
    for _ in range(n):
        if not frontier:
            break
        p = frontier.pop(draw(st.integers(0, len(frontier) - 1)))
        paths.add(p)
        if len(p) < K:
            frontier.extend(p + (i,) for i in range(k))
    order = draw(st.permutations(sorted(paths)))
    return [list(p) for p in order], K, k


@settings(max_examples=60, deadline=None)
@given(prefix_closed_trees())
def test_mask_equals_brute_force_ancestors(case):
    paths, K, k = case
    t = oracle.build_tree(paths, K, k)
    # brute force: walk parent pointers (not the prefix test used by build_tree)
    for j in range(t["T"]):
        anc = set()
        i = j
        while i != -1:
            anc.add(i)
            i = int(t["parent"][i])
        bits = {i for i in range(t["T"]) if (int(t["mask"][j, i // 64]) >> (i % 64)) & 1}
        assert bits == anc
        assert len(anc) == t["depth"][j] + 1
    # parents precede children, so one forward scan sees every parent first
    assert all(t["parent"][j] < j for j in range(1, t["T"]))
    # retrieve rows are root..leaf chains ending at a node without children
    kids = set(t["parent"][1:].tolist())
    for row in t["retrieve"]:
        ids = [int(x) for x in row if x >= 0]
        assert ids[0] == 0 and ids[-1] not in kids
        for a, b in zip(ids, ids[1:]):
            assert t["parent"][b] == a


def test_chain_mask_is_lower_triangular():
    K = 6
    paths = [[0] * d for d in range(1, K + 1)]
    t = oracle.build_tree(paths, K, 1)
    dense = np.array([[(int(t["mask"][j, 0]) >> i) & 1 for i in range(t["T"])] for j in range(t["T"])])
    assert np.array_equal(dense, np.tril(np.ones((K + 1, K + 1), dtype=int)))


def test_mask_words_beyond_64_nodes():
    t = oracle.build_tree(oracle.dense_paths(4, 4), 4, 4)
    last = t["T"] - 1                       # deepest, last leaf (3,3,3,3)
    anc = oracle.ancestors(t, last)
    assert len(anc) == 5 and anc[0] == 0
    bits = [i for i in range(t["T"]) if (int(t["mask"][last, i // 64]) >> (i % 64)) & 1]
    assert bits == anc


def test_tree_tokens_and_positions():
    t = oracle.build_tree(GOLD["two_heads_top2"]["paths"], 2, 2)
    root = np.array([7, 8])
    idx = np.array([[[10, 11], [20, 21]], [[30, 31], [40, 41]]])  # [K][B][k]
    tok = oracle.tree_tokens(t, root, idx)
    # nodes: root, (0), (1), (0,0), (0,1), (1,0), (1,1)
    assert tok.tolist() == [[7, 10, 11, 30, 31, 30, 31], [8, 20, 21, 40, 41, 40, 41]]
    assert oracle.tree_positions(t, 100).tolist() == [100, 101, 101, 102, 102, 102, 102]


def test_greedy_tie_reading_shorter_path_first():
    # a(0,0)=1/2, a(0,1)=1/4, a(1,0)=1/2: paths (1,) and (0,0) both score 1/4.
    # Reading for equal gains: the shorter path is added first.
    acc = lambda d, i: Fraction(1, 2) if (d, i) in ((0, 0), (1, 0)) else Fraction(1, 4) if (d, i) == (0, 1) else Fraction(1, 64)
    assert oracle.greedy_paths(acc, 2, 2, 2) == [(0,), (1,)]
    assert oracle.greedy_paths(acc, 2, 3, 2) == [(0,), (1,), (0, 0)]

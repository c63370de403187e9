"""Pins for the oracle's KV-cache commit (CPU only)."""
import math

import numpy as np
from scipy.special import softmax

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def tree_and_inputs(B=3, nh=2, dh=8, L_cap=40, seed=0):
    tree = oracle.build_tree(oracle.dense_paths(3, 2), 3, 2)
    T = tree["T"]
    kt, vt = rnd((B, T, nh, dh), seed), rnd((B, T, nh, dh), seed + 1)
    kc, vc = rnd((B, nh, L_cap, dh), seed + 2), rnd((B, nh, L_cap, dh), seed + 3)
    return tree, kt, vt, kc, vc


def test_committed_cache_reproduces_tree_attention_of_best():
    # the point of the commit: after it, plain decode attention of best's
    # query over the cache (prefix + root .. parent(best)) plus best itself
    # is exactly best's tree attention of the step that accepted it
    tree, kt, vt, kc, vc = tree_and_inputs(seed=5)
    B, T, nh, dh = kt.shape
    q = rnd((B, T, nh, dh), 9)
    L = np.array([7, 0, 12])
    best = np.array([T - 1, 3, 0])
    tree_out = np.stack([oracle.tree_attention(q[b:b + 1], kt[b:b + 1], vt[b:b + 1], kc[b:b + 1, :, :L[b]],
                                               vc[b:b + 1, :, :L[b]], tree)[0] for b in range(B)])
    kc2, vc2, L2 = oracle.kv_commit(tree, kt, vt, best, L, kc, vc)
    for b in range(B):
        j = best[b]
        assert L2[b] == L[b] + tree["depth"][j] + 1
        for h in range(nh):
            keys, vals = kc2[b, h, :L2[b]], vc2[b, h, :L2[b]]
            # best's own row is the last committed one
            assert np.array_equal(keys[-1], kt[b, j, h]) and np.array_equal(vals[-1], vt[b, j, h])
            ref = softmax(keys @ q[b, j, h] / math.sqrt(dh)) @ vals
            assert np.allclose(tree_out[b, j, h], ref, rtol=1e-12, atol=1e-12)


def test_chain_tree_appends_rows_in_order():
    D = 4
    tree = oracle.build_tree([[0] * d for d in range(1, D + 1)], D, 1)
    B, nh, dh, L_cap = 1, 2, 4, 10
    kt = np.arange(B * (D + 1) * nh * dh, dtype=np.float64).reshape(B, D + 1, nh, dh)
    vt = -kt
    kc = np.full((B, nh, L_cap, dh), 0.5)
    vc = np.full((B, nh, L_cap, dh), 0.25)
    kc2, vc2, L2 = oracle.kv_commit(tree, kt, vt, [3], [2], kc, vc)
    assert L2.tolist() == [6]
    for i in range(4):                      # nodes 0..3 at positions 2..5
        assert np.array_equal(kc2[0, :, 2 + i], kt[0, i]) and np.array_equal(vc2[0, :, 2 + i], vt[0, i])
    untouched = [0, 1, 6, 7, 8, 9]
    assert np.array_equal(kc2[0, :, untouched], kc[0, :, untouched])
    assert np.array_equal(vc2[0, :, untouched], vc[0, :, untouched])


def test_positions_match_tree_positions_and_other_rows_untouched():
    tree, kt, vt, kc, vc = tree_and_inputs(seed=1)
    B = kt.shape[0]
    L = np.array([3, 9, 20])
    for j in range(tree["T"]):
        best = np.full(B, j)
        kc2, _, L2 = oracle.kv_commit(tree, kt, vt, best, L, kc, vc)
        for b in range(B):
            pos = oracle.tree_positions(tree, L[b])
            path = oracle.ancestors(tree, j)
            for node in path:
                assert np.array_equal(kc2[b, :, pos[node]], kt[b, node])
            written = {int(pos[n]) for n in path}
            assert written == set(range(L[b], L2[b]))
            keep = [p for p in range(kc.shape[2]) if p not in written]
            assert np.array_equal(kc2[b][:, keep], kc[b][:, keep])


def test_capacity_and_invalid_sequences():
    tree, kt, vt, kc, vc = tree_and_inputs(L_cap=10, seed=2)
    T = tree["T"]
    deep = int(np.argmax(tree["depth"]))      # depth 3: four rows
    # 8 + 4 rows > 10: only two fit; -1 and T are not nodes; length 11 > L_cap
    best = np.array([deep, -1, T])
    L = np.array([8, 4, 4])
    kc2, vc2, L2 = oracle.kv_commit(tree, kt, vt, best, L, kc, vc)
    assert L2.tolist() == [10, 4, 4]
    path = oracle.ancestors(tree, deep)
    assert np.array_equal(kc2[0, :, 8], kt[0, path[0]]) and np.array_equal(kc2[0, :, 9], kt[0, path[1]])
    assert np.array_equal(kc2[1:], kc[1:]) and np.array_equal(vc2[1:], vc[1:])
    kc3, _, L3 = oracle.kv_commit(tree, kt, vt, np.array([0, 0, 0]), np.array([11, 10, 0]), kc, vc)
    assert L3.tolist() == [11, 10, 1] and np.array_equal(kc3[:2], kc[:2])

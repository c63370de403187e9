"""The library's host-side tree code built as plain C++ with the address and
undefined-behaviour sanitizers (tests/host_check/tree_check.cpp drives
speculative_decoding_05_amd/csrc/tree.cpp), fed page trees, dense and greedy
trees, random prefix-closed trees and invalid inputs.  Any sanitizer report
aborts the driver; every array it prints is compared with the oracle's."""
import os
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from speculative_decoding_05_amd import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = [os.path.join(ROOT, "speculative_decoding_05_amd", "csrc", "tree.cpp"),
       os.path.join(ROOT, "tests", "host_check", "tree_check.cpp")]
EXE = os.path.join(ROOT, "_build", "tree_check_san")
ENV = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


@pytest.fixture(scope="module")
def driver():
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++ on this machine")
    os.makedirs(os.path.dirname(EXE), exist_ok=True)
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-static-libasan", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "speculative_decoding_05_amd", "csrc")] + SRC + ["-o", EXE]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return EXE


def run(exe, lines):
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=ENV, timeout=300)
    assert r.returncode == 0 and "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    out = r.stdout.strip().splitlines()
    assert len(out) == len(lines)
    return [dict(kv.split("=", 1) for kv in ln.split()) for ln in out]


def tree_cmd(paths, K, k):
    parts = [f"tree {K} {k} {len(paths)}"]
    for p in paths:
        parts.append(" ".join(str(x) for x in [len(p), *p]))
    return "  ".join(parts)


def ints(s):
    return [int(x) for x in s.split(",")] if s else []


def check_tree(rec, paths, K, k):
    assert rec["status"] == "0"
    o = oracle.build_tree(paths, K, k)
    T, W = int(rec["T"]), int(rec["W"])
    assert (T, W, int(rec["D"]), int(rec["leaves"])) == (o["T"], o["W"], o["depth_max"], o["n_leaves"])
    mask = np.array([int(x, 16) for x in rec["mask"].split(",")], dtype=np.uint64).reshape(T, W)
    assert np.array_equal(mask, o["mask"])
    assert ints(rec["parent"]) == o["parent"].tolist()
    assert ints(rec["depth"]) == o["depth"].tolist()
    assert ints(rec["rank"]) == o["rank"].tolist()
    assert ints(rec["retrieve"]) == o["retrieve"].reshape(-1).tolist()
    assert ints(rec["pos100"]) == oracle.tree_positions(o, 100).tolist()


def parse_paths(rec):
    if not rec["paths"]:
        return []
    return [tuple(int(x) for x in p.split(".")) for p in rec["paths"].split(";")]


def test_config_and_dense_trees(driver):
    cases = []
    for name in configs.ORDER:
        cfg = configs.CONFIGS[name]
        spec = cfg.tree
        paths = (oracle.dense_paths(cfg.K, spec.k) if spec.kind == "dense"
                 else oracle.greedy_paths(configs.acc_exact, cfg.K, spec.n_paths, spec.rank_cap))
        cases.append((paths, cfg.K, spec.k))
    cases += [(oracle.dense_paths(K, k), K, k) for K, k in [(2, 2), (4, 2), (4, 3), (3, 6), (1, 64)]]
    cases += [([[0]], 1, 1), ([], 3, 2), ([[i] for i in range(64)] + [[0, j] for j in range(64)], 2, 64)]
    recs = run(driver, [tree_cmd(p, K, k) for p, K, k in cases])
    for rec, (p, K, k) in zip(recs, cases):
        check_tree(rec, p, K, k)


def test_dense_and_greedy_path_lists(driver):
    acc5 = " ".join(repr(configs.acc_float(d, i)) for d in range(5) for i in range(10))
    acc4 = " ".join(repr(configs.acc_float(d, i)) for d in range(4) for i in range(10))
    recs = run(driver, ["dense 2 2", "dense 4 4", "dense 3 6", f"greedy 4 10 63 {acc4}", f"greedy 5 10 63 {acc5}",
                        f"greedy 4 10 255 {acc4}"])
    assert parse_paths(recs[0]) == [tuple(p) for p in oracle.dense_paths(2, 2)]
    assert parse_paths(recs[1]) == [tuple(p) for p in oracle.dense_paths(4, 4)]
    assert parse_paths(recs[2]) == [tuple(p) for p in oracle.dense_paths(3, 6)]
    for rec, (K, n) in zip(recs[3:], [(4, 63), (5, 63), (4, 255)]):
        assert parse_paths(rec) == [tuple(p) for p in oracle.greedy_paths(configs.acc_exact, K, n, 10)]


@st.composite
def trees(draw):
    K = draw(st.integers(1, 5))
    k = draw(st.integers(1, 8))
    n = draw(st.integers(0, 400))
    paths, frontier = set(), [(i,) for i in range(k)]
    for _ in range(n):
        if not frontier:
            break
        p = frontier.pop(draw(st.integers(0, len(frontier) - 1)))
        paths.add(p)
        if len(p) < K:
            frontier.extend(p + (i,) for i in range(k))
    return [list(p) for p in draw(st.permutations(sorted(paths)))], K, k


@settings(max_examples=40, deadline=None)
@given(st.lists(trees(), min_size=1, max_size=8))
def test_random_prefix_closed_trees(driver, cases):
    recs = run(driver, [tree_cmd(p, K, k) for p, K, k in cases])
    for rec, (p, K, k) in zip(recs, cases):
        check_tree(rec, p, K, k)


def test_invalid_trees_and_arguments(driver):
    big = [[i] for i in range(64)] + [[i, j] for i in range(64) for j in range(16)]     # T = 1089
    cases = [
        ([[0, 0]], 2, 2, 3),                 # missing prefix
        ([[0], [0]], 2, 2, 3),               # duplicate
        ([[2]], 2, 2, 3),                    # rank >= k
        ([[-1]], 2, 2, 3),                   # negative rank
        ([[0], [0, 0], [0, 0, 0]], 2, 2, 3),  # longer than K
        ([[]], 2, 2, 3),                     # empty path
        ([[0]], 1, 65, 4),                   # k above the limit
        (big, 2, 64, 4),                     # T above the limit
    ]
    recs = run(driver, [tree_cmd(p, K, k) for p, K, k, _ in cases] + ["errors"])
    for rec, (_, _, _, code) in zip(recs, cases):
        assert int(rec["status"]) == code
    # NULL / out-of-range arguments of the host calls, in the driver's order
    assert ints(recs[-1]["codes"]) == [1, 1, 1, 1, 4, 1, 1, 1, 4, 1, 1, 1, 3, 4]

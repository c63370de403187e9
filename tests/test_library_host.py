"""The C-ABI library on the CPU: exported symbols, host-side tree building
(bit-exact against the oracle) and argument validation.  No kernel runs."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from speculative_decoding_05_amd import configs
from tests._lib import mb

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "medusa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)) - {"sizeof"}


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 18
    assert names == set(mb.SIGNATURES)
    for n in names:
        assert hasattr(mb.lib, n)
    assert mb.lib.medusa_abi_version() == 1


def same_tree(t, o):
    assert t.T == o["T"] and t.W == o["W"] and t.depth_max == o["depth_max"] and t.n_leaves == o["n_leaves"]
    assert np.array_equal(t.mask, o["mask"])
    assert t.parent.tolist() == o["parent"].tolist()
    assert t.depth.tolist() == o["depth"].tolist()
    assert t.rank.tolist() == o["rank"].tolist()
    assert t.retrieve.tolist() == o["retrieve"].tolist()


@pytest.mark.parametrize("K,k", [(2, 2), (4, 2), (4, 3), (4, 4), (1, 7), (3, 5)])
def test_dense_paths_and_tree_match_oracle(K, k):
    paths = mb.dense_paths(K, k)
    assert paths == oracle.dense_paths(K, k)
    same_tree(mb.Tree(paths, K, k), oracle.build_tree(paths, K, k))


@pytest.mark.parametrize("K", [4, 5])
def test_greedy_paths_match_oracle(K):
    acc = np.array([[configs.acc_float(d, i) for i in range(10)] for d in range(K)])
    got = mb.greedy_paths(acc, 63)
    assert got == oracle.greedy_paths(configs.acc_exact, K, 63, 10)
    same_tree(mb.Tree(got, K, 10), oracle.build_tree(got, K, 10))


def test_config_trees():
    for name in configs.ORDER:
        cfg = configs.CONFIGS[name]
        spec = cfg.tree
        if spec.kind == "dense":
            paths = oracle.dense_paths(cfg.K, spec.k)
        else:
            paths = oracle.greedy_paths(configs.acc_exact, cfg.K, spec.n_paths, spec.rank_cap)
        t = mb.Tree(paths, cfg.K, spec.k)
        assert t.T == {"tiny_f32": 7, "dense341_b32": 341}.get(name, 64)
        assert t.positions(cfg.L).tolist() == (cfg.L + t.depth).tolist()


@st.composite
def trees(draw):
    K = draw(st.integers(1, 5))
    k = draw(st.integers(1, 6))
    n = draw(st.integers(0, 150))
    paths, frontier = set(), [(i,) for i in range(k)]
    for _ in range(n):
        if not frontier:
            break
        p = frontier.pop(draw(st.integers(0, len(frontier) - 1)))
        paths.add(p)
        if len(p) < K:
            frontier.extend(p + (i,) for i in range(k))
    return draw(st.permutations(sorted(paths))), K, k


@settings(max_examples=80, deadline=None)
@given(trees())
def test_random_trees_bit_exact(case):
    paths, K, k = case
    same_tree(mb.Tree(paths, K, k), oracle.build_tree(paths, K, k))


@pytest.mark.parametrize("paths,K,k,code", [
    ([[0, 0]], 2, 2, mb.ERR_TREE),
    ([[0], [0]], 2, 2, mb.ERR_TREE),
    ([[2]], 2, 2, mb.ERR_TREE),
    ([[0], [0, 0], [0, 0, 0]], 2, 2, mb.ERR_TREE),
    ([[]], 2, 2, mb.ERR_TREE),
    ([[-1]], 2, 2, mb.ERR_TREE),
    ([[0]], 1, 65, mb.ERR_UNSUPPORTED),
])
def test_invalid_trees_return_codes(paths, K, k, code):
    with pytest.raises(mb.MedusaError) as e:
        mb.Tree(paths, K, k)
    assert e.value.status == code


def test_tree_size_limit():
    with pytest.raises(mb.MedusaError) as e:
        mb.dense_paths(5, 4)                    # 1364 paths > 1023
    assert e.value.status == mb.ERR_UNSUPPORTED
    paths = [(i,) for i in range(64)] + [(i, j) for i in range(64) for j in range(16)]
    with pytest.raises(mb.MedusaError) as e:
        mb.Tree(paths, 2, 64)                   # T = 1089
    assert e.value.status == mb.ERR_UNSUPPORTED


def test_device_calls_validate_before_launch():
    # every case below is rejected by host-side checks; no HIP call is made
    t = mb.Tree([[0], [1]], 1, 2)               # not uploaded
    P = ctypes.c_void_p
    fake = P(0x1000)
    s = mb.lib.tree_attention(None, mb.BF16, t.handle, 1, 1, 128, 8, 0.0, fake, fake, fake, fake, fake,
                              fake, None, 0)
    assert s == mb.ERR_STATE
    s = mb.lib.typical_accept(None, t.handle, 1, 10, fake, fake, 0.09, 0.3, 1.0, fake, fake, fake, fake,
                              None, None, fake, 1 << 20)
    assert s == mb.ERR_STATE
    assert mb.lib.medusa_topk(None, 2, 10, 11, fake, fake, None, fake, 1 << 20) == mb.ERR_ARG
    assert mb.lib.medusa_topk(None, 2, 100, 65, fake, fake, None, fake, 1 << 20) == mb.ERR_UNSUPPORTED
    assert mb.lib.medusa_topk(None, 2, 40000, 4, fake, fake, None, fake, 8) == mb.ERR_WORKSPACE
    assert mb.lib.medusa_pack_weights(None, 2, 10, 100, 1, fake, fake) == mb.ERR_UNSUPPORTED
    assert mb.lib.medusa_pack_weights(None, 2, 10, 128, 3, fake, fake) == mb.ERR_ARG      # group not a power of 2
    assert mb.lib.medusa_head_vocab_packed(None, 2, 1, 128, 10, 16, fake, fake, fake) == mb.ERR_ARG
    assert mb.lib.medusa_heads_packed(None, 4, 1, 256, 0, 1, fake, fake, fake, fake, fake) == mb.ERR_ARG
    assert [mb.medusa_pack_group_for_rows(m) for m in (1, 8, 9, 32, 1000)] == [1, 1, 8, 8, 8]
    assert mb.lib.medusa_heads(None, mb.BF16, 4, 1, 100, 50, fake, fake, fake, fake, fake) == mb.ERR_UNSUPPORTED
    assert mb.lib.medusa_heads(None, mb.BF16, 4, 1, 256, 50, fake, None, fake, fake, fake) == mb.ERR_ARG
    assert mb.lib.medusa_heads(None, mb.BF16, 4, 1, 256, 50, P(0x1008), fake, fake, fake, fake) == mb.ERR_ARG
    assert b"aligned" in mb.lib.medusa_last_error()
    assert mb.lib.medusa_tree_tokens(None, t.handle, 1, 1, 2, fake, fake, fake) == mb.ERR_STATE


def test_head_workspace_calls_reject_bad_arguments_before_launch():
    P = ctypes.c_void_p
    fake = P(0x1000)
    need = mb.medusa_head_workspace(2, 100, 256)
    # M >= 65: workspace checks come before anything is enqueued
    assert mb.lib.medusa_head_vocab_packed_ws(None, 2, 100, 256, 500, 8, fake, fake, fake, fake, need - 1) \
        == mb.ERR_WORKSPACE
    assert mb.lib.medusa_head_vocab_packed_ws(None, 2, 100, 256, 500, 8, fake, fake, fake, None, need) == mb.ERR_ARG
    assert mb.lib.medusa_head_vocab_packed_ws(None, 2, 100, 256, 500, 8, fake, fake, fake, P(0x1008), need) \
        == mb.ERR_ARG
    assert b"aligned" in mb.lib.medusa_last_error()
    assert mb.lib.medusa_head_resblock_packed_ws(None, 2, 100, 256, 3, fake, fake, fake, fake, need) == mb.ERR_ARG
    assert mb.lib.medusa_head_resblock_packed_ws(None, 2, 100, 256, 8, fake, fake, None, fake, need) == mb.ERR_ARG
    assert mb.lib.medusa_head_resblock_packed_ws(None, 2, 100, 256, 8, fake, fake, fake, fake, 16) \
        == mb.ERR_WORKSPACE
    assert mb.lib.medusa_head_vocab_packed_ws(None, 2, 100, 256, 0, 8, fake, fake, fake, fake, need) == mb.ERR_ARG


def test_heads_combined_workspace_call_rejects_bad_arguments_before_launch():
    P = ctypes.c_void_p
    fake = P(0x1000)
    need = mb.medusa_heads_workspace(2, 100, 256)
    assert need == mb.medusa_head_workspace(3, 100, 256)          # packed h + packed r of 2 heads
    args = [None, 2, 100, 256, 500, 8, fake, fake, fake, fake, fake]
    assert mb.lib.medusa_heads_packed_ws(*args, fake, need - 16) == mb.ERR_WORKSPACE
    assert mb.lib.medusa_heads_packed_ws(*args, None, need) == mb.ERR_ARG
    assert mb.lib.medusa_heads_packed_ws(*args, P(0x1008), need) == mb.ERR_ARG
    assert mb.lib.medusa_heads_packed_ws(None, 2, 100, 256, 500, 5, fake, fake, fake, fake, fake, fake, need) \
        == mb.ERR_ARG
    assert mb.lib.medusa_heads_packed_ws(None, 2, 100, 256, 500, 8, fake, fake, None, fake, fake, fake, need) \
        == mb.ERR_ARG
    assert mb.medusa_heads_workspace(4, 64, 4096) == 0
    assert mb.medusa_heads_workspace(4, 1024, 4096) == 5 * 64 * 128 * 1024


def test_head_workspace_calls_check_shape_limits_before_launch():
    # one head's packed activations over 4 GiB: refused as unsupported before any
    # launch (on this host a launch would fail with ERR_HIP instead)
    P = ctypes.c_void_p
    fake = P(0x1000)
    M, H = 600000, 4096                      # 37500 row tiles x 128 KiB = 4.6 GiB per head
    huge = 1 << 40
    assert mb.lib.medusa_head_vocab_packed_ws(None, 1, M, H, 1000, 8, fake, fake, fake, fake, huge) \
        == mb.ERR_UNSUPPORTED
    assert b"4 GiB" in mb.lib.medusa_last_error()
    assert mb.lib.medusa_head_resblock_packed_ws(None, 1, M, H, 8, fake, fake, fake, fake, huge) \
        == mb.ERR_UNSUPPORTED
    assert mb.lib.medusa_heads_packed_ws(None, 1, M, H, 1000, 8, fake, fake, fake, fake, fake, fake, huge) \
        == mb.ERR_UNSUPPORTED


def test_head_workspace_size():
    # activations in fragment order: K * ceil(M/16) * (H/32) KiB, from 65 rows on
    assert mb.medusa_head_workspace(4, 64, 4096) == 0
    assert mb.medusa_head_workspace(4, 65, 4096) == 4 * 5 * 128 * 1024
    assert mb.medusa_head_workspace(4, 1024, 4096) == 4 * 64 * 128 * 1024
    assert mb.medusa_head_workspace(5, 512, 5120) == 5 * 32 * 160 * 1024
    assert mb.medusa_head_workspace(1, 10912, 4096) == 682 * 128 * 1024
    assert mb.medusa_head_workspace(2, 100, 100) == 0                  # H % 128 != 0
    assert mb.medusa_head_workspace(0, 100, 256) == 0


def test_workspace_sizes():
    assert mb.medusa_topk_workspace(64, 32000, 10) == 0              # one slice per row
    assert mb.medusa_topk_workspace(4, 70000, 10) == 4 * 3 * 10 * 8   # three sorted lists per row
    t = mb.Tree(oracle.dense_paths(2, 2), 2, 2)
    assert mb.typical_accept_workspace(t, 3, 1000) == 3 * 3 * 1 * 32 + 3 * 16   # 3 internal rows, 1 chunk; scan slots


def test_injected_launch_failure_returns_err_hip_before_launch(monkeypatch):
    # MEDUSA_FAULT=launch fails every launch before it is enqueued, so these
    # argument-valid calls return ERR_HIP without touching the (fake) buffers
    P = ctypes.c_void_p
    fake = P(0x1000)
    monkeypatch.setenv("MEDUSA_FAULT", "launch")
    assert mb.lib.medusa_heads(None, mb.BF16, 4, 1, 256, 64, fake, fake, fake, fake, fake) == mb.ERR_HIP
    assert b"injected" in mb.lib.medusa_last_error()
    assert mb.lib.medusa_topk(None, 2, 1000, 4, fake, fake, None, None, 0) == mb.ERR_HIP
    assert mb.lib.medusa_pack_weights(None, 2, 10, 128, 1, fake, fake) == mb.ERR_HIP
    # argument errors still win over the injected failure
    assert mb.lib.medusa_topk(None, 2, 1000, 65, fake, fake, None, None, 0) == mb.ERR_UNSUPPORTED


def test_trace_mode_runs_without_a_profiler():
    # MEDUSA_TRACE=1 opens roctx at run time and wraps the call in a range; with
    # no profiler attached the call behaves as without it (here: the injected
    # launch failure).  A child process, since the switch is read once.
    import subprocess
    import sys
    code = ("import ctypes; from tests._lib import mb; f = ctypes.c_void_p(0x1000); "
            "s = mb.lib.medusa_heads(None, mb.BF16, 4, 1, 256, 64, f, f, f, f, f); "
            "print(s, mb.lib.medusa_last_error().decode())")
    env = dict(os.environ, MEDUSA_TRACE="1", MEDUSA_FAULT="launch", HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(__file__)), env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert r.stdout.split()[0] == str(mb.ERR_HIP) and "injected" in r.stdout

"""Debug modes of the library on the GPU: MEDUSA_VALIDATE=1 (NaN / +inf logits
give ERR_NONFINITE, token ids outside [0, V) give ERR_ARG, outputs untouched;
clean inputs give the same results as without it), and MEDUSA_FAULT=launch on
real buffers (ERR_HIP, nothing enqueued).  Also the greedy-threshold and
root-only-tree cases of acceptance and the fused top-k."""
import numpy as np
import pytest
import torch

import oracle
from speculative_decoding_05_amd import configs, synth
from tests._lib import mb
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def accept_inputs(B=3, V=2000, seed=4):
    paths = oracle.dense_paths(3, 3)
    ot = oracle.build_tree(paths, 3, 3)
    t = mb.Tree(paths, 3, 3).upload()
    g = np.random.default_rng(seed)
    idx = np.stack([np.stack([g.choice(V, 3, replace=False) for _ in range(B)]) for _ in range(3)])
    root = g.integers(0, V, B)
    tok = oracle.tree_tokens(ot, root, idx)
    vl = synth.verification_logits(900 + seed, V, ot["parent"], ot["depth"], ot["rank"], idx, root,
                                   configs.acc_float, 3)
    head = (g.standard_normal((3, B, V)) * 2).astype(np.float32)
    return ot, t, tok.astype(np.int32), vl, head


def outputs(B, D):
    o = {n: torch.full((B,), -9, dtype=torch.int32, device="cuda") for n in ("len", "best", "next")}
    o["acc"] = torch.full((B, D + 1), -9, dtype=torch.int32, device="cuda")
    return o


def typical(t, vl, tok, o, ws):
    mb.typical_accept(t, vl, tok, 0.09, 0.3, 1.0, o["len"], o["best"], o["next"], o["acc"], ws=ws)


def untouched(o):
    torch.cuda.synchronize()
    return all(bool((v == -9).all()) for v in o.values())


def test_validate_typical_accept(monkeypatch):
    ot, t, tok, vl, _ = accept_inputs()
    B, T, V = vl.shape
    ws = mb.workspace(mb.typical_accept_workspace(t, B, V))
    d_tok = dev(tok)
    # clean inputs: the same results with and without validation
    ref = outputs(B, ot["depth_max"])
    typical(t, dev(vl), d_tok, ref, ws)
    monkeypatch.setenv("MEDUSA_VALIDATE", "1")
    got = outputs(B, ot["depth_max"])
    typical(t, dev(vl), d_tok, got, ws)
    for n in ref:
        assert torch.equal(ref[n], got[n]), n
    for bad_value in (np.nan, np.inf):
        x = vl.copy()
        x[B - 1, T - 1, V // 2] = bad_value
        o = outputs(B, ot["depth_max"])
        with pytest.raises(mb.MedusaError) as e:
            typical(t, dev(x), d_tok, o, ws)
        assert e.value.status == mb.ERR_NONFINITE
        assert untouched(o)
    x = vl.copy()
    x[0, 0, 3] = -np.inf                     # -inf is allowed
    typical(t, dev(x), d_tok, outputs(B, ot["depth_max"]), ws)
    for bad_tok in (V, -1):
        bt = tok.copy()
        bt[1, 5] = bad_tok
        o = outputs(B, ot["depth_max"])
        with pytest.raises(mb.MedusaError) as e:
            typical(t, dev(vl), dev(bt), o, ws)
        assert e.value.status == mb.ERR_ARG
        assert untouched(o)


def test_validate_topk_and_tree_tokens(monkeypatch):
    K, B, V, k = 3, 2, 5000, 4
    paths = oracle.dense_paths(3, 2)
    t = mb.Tree(paths, K, 2).upload()
    g = np.random.default_rng(7)
    x = g.standard_normal((K, B, V)).astype(np.float32)
    root = g.integers(0, V, B).astype(np.int32)
    monkeypatch.setenv("MEDUSA_VALIDATE", "1")
    idx = torch.full((K, B, k), -9, dtype=torch.int32, device="cuda")
    tok = torch.full((B, t.T), -9, dtype=torch.int32, device="cuda")
    mb.medusa_topk_tree_tokens(t, dev(x), k, dev(root), idx, tok)
    assert np.array_equal(host(idx), oracle.topk_per_head(x.astype(np.float64), k)[0])
    xn = x.copy()
    xn[2, 1, 17] = np.nan
    for fn in (lambda: mb.medusa_topk(dev(xn.reshape(K * B, V)), k, idx.reshape(K * B, k)),
               lambda: mb.medusa_topk_tree_tokens(t, dev(xn), k, dev(root), idx, tok)):
        idx.fill_(-9)
        tok.fill_(-9)
        with pytest.raises(mb.MedusaError) as e:
            fn()
        assert e.value.status == mb.ERR_NONFINITE
        torch.cuda.synchronize()
        assert bool((idx == -9).all()) and bool((tok == -9).all())
    xi = x.copy()
    xi[0, 0, :2] = [np.inf, -np.inf]          # +-inf are ordered values for top-k
    mb.medusa_topk(dev(xi.reshape(K * B, V)), k, idx.reshape(K * B, k))
    assert host(idx)[0, 0, 0] == 0
    bad_root = root.copy()
    bad_root[1] = V
    with pytest.raises(mb.MedusaError) as e:
        mb.medusa_topk_tree_tokens(t, dev(x), k, dev(bad_root), idx, tok)
    assert e.value.status == mb.ERR_ARG


def test_validate_rejection_accept(monkeypatch):
    ot, t, tok, vl, head = accept_inputs(seed=5)
    B, T, V = vl.shape
    g = np.random.default_rng(1)
    u_node, u_bonus = dev(g.random((B, T)).astype(np.float32)), dev(g.random(B).astype(np.float32))
    monkeypatch.setenv("MEDUSA_VALIDATE", "1")
    o = outputs(B, ot["depth_max"])
    mb.rejection_accept(t, dev(vl), dev(head), dev(tok), 1.0, u_node, u_bonus, o["len"], o["best"], o["next"],
                        o["acc"])
    hn = head.copy()
    hn[1, 2, 9] = np.nan
    o = outputs(B, ot["depth_max"])
    with pytest.raises(mb.MedusaError) as e:
        mb.rejection_accept(t, dev(vl), dev(hn), dev(tok), 1.0, u_node, u_bonus, o["len"], o["best"], o["next"],
                            o["acc"])
    assert e.value.status == mb.ERR_NONFINITE
    assert untouched(o)


def test_injected_launch_failure_on_real_buffers(monkeypatch):
    ot, t, tok, vl, _ = accept_inputs(seed=6)
    B, T, V = vl.shape
    ws = mb.workspace(mb.typical_accept_workspace(t, B, V))
    monkeypatch.setenv("MEDUSA_FAULT", "launch")
    o = outputs(B, ot["depth_max"])
    with pytest.raises(mb.MedusaError) as e:
        typical(t, dev(vl), dev(tok), o, ws)
    assert e.value.status == mb.ERR_HIP and "injected" in str(e.value)
    assert untouched(o)
    monkeypatch.delenv("MEDUSA_FAULT")
    typical(t, dev(vl), dev(tok), o, ws)
    torch.cuda.synchronize()
    assert not untouched(o)


def test_greedy_acceptance_respects_the_threshold():
    # temperature 0: p is one-hot at the argmax, H = 0, threshold min(eps, delta);
    # with eps = delta = 1 no candidate clears it (1 > 1 is false), as in the oracle
    ot, t, tok, vl, _ = accept_inputs(seed=8)
    B, T, V = vl.shape
    ws = mb.workspace(mb.typical_accept_workspace(t, B, V))
    # make every depth-1 candidate the argmax of the root row, so that only the threshold decides
    x = vl.copy()
    for b in range(B):
        x[b, 0, tok[b, 1]] = x[b, 0].max() + 5.0
    for eps, delta in ((1.0, 1.0), (0.09, 0.3)):
        o = outputs(B, ot["depth_max"])
        cp = torch.empty((B, T), dtype=torch.float32, device="cuda")
        th = torch.empty((B, T), dtype=torch.float32, device="cuda")
        mb.typical_accept(t, dev(x), dev(tok), eps, delta, 0.0, o["len"], o["best"], o["next"], o["acc"], cp, th,
                          ws=ws)
        ref = oracle.typical_accept(x.astype(np.float64), tok, ot, eps, delta, 0.0)
        assert host(o["len"]).tolist() == ref["accept_len"].tolist(), (eps, delta)
        assert host(o["best"]).tolist() == ref["best"].tolist(), (eps, delta)
        assert np.allclose(host(th)[:, 0], min(eps, delta))
        if eps == 1.0:
            assert (host(o["len"]) == 0).all()
        else:
            assert (host(o["len"]) >= 1).all()


def test_topk_tree_tokens_root_only_tree():
    # a tree of the root alone: the fused call still writes every root token
    t = mb.Tree([], 2, 3).upload()
    K, B, V, k = 2, 4, 1000, 3
    g = np.random.default_rng(9)
    x = g.standard_normal((K, B, V)).astype(np.float32)
    root = g.integers(0, V, B).astype(np.int32)
    idx = torch.full((K, B, k), -9, dtype=torch.int32, device="cuda")
    tok = torch.full((B, 1), -9, dtype=torch.int32, device="cuda")
    mb.medusa_topk_tree_tokens(t, dev(x), k, dev(root), idx, tok)
    assert host(tok)[:, 0].tolist() == root.tolist()
    assert np.array_equal(host(idx), oracle.topk_per_head(x.astype(np.float64), k)[0])


def test_peak_kernels_run():
    # the two measurement kernels: they run, leave the sink alone (the data never
    # triggers its store), and report a plausible flop count
    buf = torch.ones(1 << 26, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    mb.peak_hbm_read(buf, sink)
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda")
    flops = mb.peak_mfma_bf16(8, 10, fsink)
    torch.cuda.synchronize()
    assert flops == 8 * 4 * 4 * 10 * 2 * 32 * 32 * 16
    assert bool((sink == 0).all()) and bool((fsink == 0).all())
    cus, clock_khz, _ = mb.device_info()
    assert cus >= 1 and clock_khz >= 0

#!/usr/bin/env python3
"""Medusa verify tree-steps per second on one MI355X.

One step = medusa heads (ResBlock + vocabulary projection) -> per-head top-k
-> tree tokens -> tree attention over the prefix cache -> typical
acceptance, over the whole batch, on synthetic seeded data of the workload's
shape (default: 7B shape, batch 1, KV 1024, 4 Medusa heads, 64-node tree).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

Prints one JSON line.  Inputs are resident in HBM before the timed region;
per-step inputs (hidden state, tree Q/K/V, KV cache, verification logits)
rotate over enough copies to exceed the 256 MB last-level cache.  The
dominant kernel's average duration is measured with HIP events recorded on
the stream it is launched on, inside the timed region (every 8th step by
default, since each event pair delays the next launch by a few microseconds).  The CPU oracle is
timed afterwards on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # MI355X HBM3E, bytes/s
BF16_PEAK = 2.5e15         # dense bf16 MFMA, flop/s
FP32_PEAK = 157.3e12       # fp32 vector (the fp32 path's contractions run on VALU), flop/s


def flop_peak(cfg):
    return BF16_PEAK if cfg.dtype == "bf16" else FP32_PEAK
METRIC = "Medusa verify tree-steps/sec at 1 GPU (64-node tree, 7B shape); % HBM roofline"


def elem(cfg):
    return 2 if cfg.dtype == "bf16" else 4


def stage_bytes(cfg, tree):
    """Algorithmic HBM bytes of each stage of one step (each tensor moved once)."""
    from speculative_decoding_05_amd import step as st
    e, B, K, H, V = elem(cfg), cfg.B, cfg.K, cfg.H, cfg.V
    n_int = len(set(tree.parent[1:].tolist()))          # nodes with children
    # with tile maxima the projection also writes one image per 16 logits and
    # the top-k reads those images plus k candidate tiles of 64 bytes per row
    tm = st.uses_tile_max(cfg)
    images = K * B * ((V + 15) // 16) * 4
    return {
        "head_resblock": K * H * H * e + B * H * e + K * B * H * e,
        "head_vocab": K * V * H * e + K * B * H * e + K * B * V * 4 + (images if tm else 0),
        "topk_tokens": images + K * B * cfg.k * 64 if tm else K * B * V * 4,
        "attention": 2 * B * cfg.nh * cfg.L * cfg.dh * e + 4 * B * tree.T * cfg.nh * cfg.dh * e,
        "accept": B * n_int * V * 4 + B * V * 4,
    }


def stage_flops(cfg, tree):
    B, K, H, V = cfg.B, cfg.K, cfg.H, cfg.V
    anc = int((tree.depth + 1).sum())
    return {
        "head_resblock": 2 * K * B * H * H,
        "head_vocab": 2 * K * B * H * V,
        "attention": 4 * B * cfg.nh * cfg.dh * (tree.T * cfg.L + anc),
    }


PROFILE = os.path.join(ROOT, "profiles", "head_vocab_vicuna7b_b1.md")
# sources the vocabulary-projection kernel is compiled from (kernel, packed
# layout helpers, shared device helpers); the recorded digest covers all three
KERNEL_SRCS = [os.path.join(ROOT, "speculative_decoding_05_amd", "csrc", f)
               for f in ("heads.hip", "gemm.h", "common.h")]


def kernel_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()


def counted_traffic(workload):
    """HBM bytes per launch of the vocabulary projection from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (scaled by the plain-copy
    calibration recorded there); None if there is none for this workload or
    the kernel sources changed since the counters were taken."""
    try:
        lines = open(PROFILE).read().splitlines()
    except OSError:
        return None
    rec = None
    for ln in lines:
        if ln.startswith("traffic: "):
            rec = json.loads(ln[len("traffic: "):])
    if not rec or rec.get("workload") != workload:
        return None
    if kernel_sources_sha256() != rec.get("source_sha256"):
        return None
    return rec["bytes_per_launch"]


def verify_pass(s, reps):
    """The dense contractions at the verify-pass shape (M = B*T rows): Medusa
    heads over every tree node and the LM head over the attention output.
    Each contraction first runs untimed for about 60 ms of sustained load (the
    chip raises its clock over the first tens of milliseconds of matrix-core
    work: measured, the 1024-row vocabulary projection goes from 1.31 to
    0.93 ms per call over its first 30 calls), then `reps` calls are timed
    with HIP events on the launch stream; matrix-core utilisation against the
    dense bf16 peak."""
    import time
    import torch
    from speculative_decoding_05_amd import step as st
    cfg = s.cfg
    vp = st.VerifyPass(s, seed=cfg.cfg_id)
    M, H, V, K = vp.M, cfg.H, cfg.V, cfg.K
    flops = {"heads_resblock": 2.0 * K * M * H * H, "heads_vocab": 2.0 * K * M * H * V,
             "heads": 2.0 * K * M * H * (H + V), "lm_head": 2.0 * M * H * V}
    # heads_resblock / heads_vocab: the two projections as separate calls; heads: both in
    # one call (the verify pass runs that one, then the LM head)
    fns = {"heads_resblock": vp.heads_resblock, "heads_vocab": vp.heads_vocab, "heads": vp.heads,
           "lm_head": vp.lm_head}
    # algorithmic HBM bytes (weights, activations and outputs once each): at few
    # rows the contractions stream weights, and this rate is the one that binds
    e = 2  # bf16
    hbm = {"heads_resblock": K * H * H * e + M * H * e * 2 + K * M * H * e,
           "heads_vocab": K * V * H * e + K * M * H * e + K * M * V * 4,
           "heads": K * (H + V) * H * e + M * H * e * 2 + K * M * H * e + K * M * V * 4,
           "lm_head": V * H * e + M * H * e + M * V * 4}
    out = {"rows": M, "us": {}, "tflops": {}, "mfma_frac": {}, "hbm_gbps": {}}
    for name, fn in fns.items():
        fn()
        torch.cuda.synchronize()
        t0, n = time.perf_counter(), 0
        while n < 3 or time.perf_counter() - t0 < 0.06:
            fn()
            torch.cuda.synchronize()
            n += 1
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        out["us"][name] = us
        out["tflops"][name] = flops[name] / (us * 1e-6) / 1e12
        out["mfma_frac"][name] = flops[name] / (us * 1e-6) / BF16_PEAK
        out["hbm_gbps"][name] = hbm[name] / (us * 1e-6) / 1e9
    tot_f = flops["heads"] + flops["lm_head"]
    tot_us = out["us"]["heads"] + out["us"]["lm_head"]
    out["total"] = {"us": tot_us, "tflops": tot_f / (tot_us * 1e-6) / 1e12,
                    "mfma_frac": tot_f / (tot_us * 1e-6) / BF16_PEAK}
    del vp
    torch.cuda.empty_cache()
    return out


def time_steps(s, n, warmup, copies=1):
    """Average us of a whole step over n steps, and per-stage us from a
    separate instrumented pass (events between stages)."""
    import torch
    for i in range(warmup):
        s.run(i % copies)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n):
        s.run(i % copies)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / n
    names = ["head_resblock", "head_vocab", "topk_tokens", "attention", "accept"]
    fns = [s.heads, s.heads_vocab, s.topk_and_tokens, s.attention, s.accept]
    reps = min(n, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record()
        for j, fn in enumerate(fns):
            fn(i % copies)
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    stage = {nm: 1e3 * sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(reps)) / reps
             for j, nm in enumerate(names)}
    return us, stage


def composed_step(s, steps, warmup, copies, seed):
    """The verify tree-step with its verification logits computed instead of
    planted: heads on the B sequences' hidden states, top-k and tree tokens,
    tree attention, then the LM head (a Medusa head with W1 = 0, seeded random
    weights) over the attention output of all M = B*T nodes, then typical
    acceptance on those logits.  The attention output stands in for the last
    hidden state of the verify forward (one attention, no backbone layers), so
    the accepted lengths mean nothing here; the time of every stage does."""
    import torch
    from speculative_decoding_05_amd import binding as mb
    from speculative_decoding_05_amd import step as st
    cfg, tree = s.cfg, s.tree
    B, T, V, H = cfg.B, tree.T, cfg.V, cfg.H
    vp = st.VerifyPass(s, seed=seed)
    vl = vp.vlogits.view(B, T, V)

    def accept_lm(i=0):
        mb.typical_accept(tree, vl, s.tree_tok, cfg.eps, cfg.delta, cfg.temperature, s.accept_len, s.best,
                          s.next_tok, s.accepted, None, None, s.ws_acc)

    def lm_head(i=0):
        vp.lm_head()

    names = ["head_resblock", "head_vocab", "topk_tokens", "attention", "lm_head", "accept"]
    fns = [s.heads, s.heads_vocab, s.topk_and_tokens, s.attention, lm_head, accept_lm]

    def one(i):
        for fn in fns:
            fn(i % copies)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        one(i)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    reps = min(steps, 50)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(reps)]
    for i in range(reps):
        evs[i][0].record()
        for j, fn in enumerate(fns):
            fn(i % copies)
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    stage = {nm: 1e3 * sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(reps)) / reps
             for j, nm in enumerate(names)}
    e = elem(cfg)
    M = B * T
    sb, sf = stage_bytes(cfg, tree), stage_flops(cfg, tree)
    sb["lm_head"] = V * H * e + M * H * e + M * V * 4
    sf["lm_head"] = 2 * M * H * V
    roof = {n: max(sb[n] / HBM_PEAK, sf.get(n, 0) / BF16_PEAK) * 1e6 for n in names}
    out = {"us_per_step": us, "tree_steps_per_s": 1e6 / us, "seq_steps_per_s": B * 1e6 / us, "steps": steps,
           "lm_head_rows": M, "stage_us": stage, "stage_roofline_us": roof,
           "step_roofline_us": sum(roof.values()), "roofline_frac_step": sum(roof.values()) / us,
           "lm_head_bound": "mfma" if sf["lm_head"] / BF16_PEAK > sb["lm_head"] / HBM_PEAK else "hbm",
           "note": "verification logits from an LM head over the tree-attention output (random weights)"}
    del vp, vl
    torch.cuda.empty_cache()
    return out


def tree_sweep(cfg, args):
    """Step time against tree size at the workload's shapes: greedy sparse
    trees of 16..256 nodes and dense trees of about 256 and 340 candidates
    (the acceptance side of the comparison needs a trained model)."""
    import dataclasses
    import torch
    from speculative_decoding_05_amd import binding as mb
    from speculative_decoding_05_amd import configs, synth
    from speculative_decoding_05_amd import step as st
    base_tree = st.build_tree(cfg)
    base = st.Step(cfg, base_tree, st.host_inputs(cfg, base_tree.T))
    variants = [("greedy", n) for n in (15, 31, 63, 127, 255)] + [("dense", (3, 6)), ("dense", (4, 4))]
    for kind, arg in variants:
        if kind == "greedy":
            spec = configs.TreeSpec("greedy", k=10, n_paths=arg, rank_cap=10)
            c2 = dataclasses.replace(cfg, tree=spec)
            tree = st.build_tree(c2)
        else:
            depth, k = arg
            spec = configs.TreeSpec("dense", k=k)
            c2 = dataclasses.replace(cfg, tree=spec)
            tree = mb.Tree(mb.dense_paths(depth, k), cfg.K, k).upload()
        host = {"h": synth.hidden(c2), "root_tok": synth.root_tokens(c2)}
        host["q"], host["kt"], host["vt"] = synth.tree_qkv(c2, tree.T)
        host["kc"], host["vc"] = synth.kv_cache(c2)
        s2 = st.Step(c2, tree, host, weights_of=base)
        s2.heads()
        s2.heads_vocab()
        s2.topk_and_tokens()
        torch.cuda.synchronize()
        s2.set_verify_logits(st.verify_logits_for(c2, tree, s2.topk_idx.cpu().numpy(), host["root_tok"]))
        us, stage = time_steps(s2, args.steps, args.warmup)
        print(json.dumps({"sweep": "trees", "workload": cfg.name, "tree": kind, "T": tree.T, "k": spec.k,
                          "depth_max": tree.depth_max, "us_per_step": us, "stage_us": stage}), flush=True)
        del s2
        torch.cuda.empty_cache()


def accept_sweep(cfg, args, n_seq=32):
    """Synthetic accept-length curves on the workload's tree: typical
    acceptance against its threshold eps (0.01..0.25) and against the
    temperature, rejection sampling against the temperature.  Candidates are
    the library's top-k of seeded head logits; verification logits are planted
    at them; uniforms are seeded.  Mean accepted candidates per step."""
    import dataclasses
    import numpy as np
    import torch
    from speculative_decoding_05_amd import binding as mb
    from speculative_decoding_05_amd import step as st
    from speculative_decoding_05_amd import synth
    c2 = dataclasses.replace(cfg, B=n_seq)
    tree = st.build_tree(c2)
    B, T, V, K, k = n_seq, tree.T, cfg.V, cfg.K, cfg.k
    g = torch.Generator(device="cuda").manual_seed(cfg.cfg_id)
    head = torch.randn((K, B, V), generator=g, device="cuda") * 2.5
    root = torch.from_numpy(synth.root_tokens(c2)).cuda()
    idx = torch.empty((K, B, k), dtype=torch.int32, device="cuda")
    tok = torch.empty((B, T), dtype=torch.int32, device="cuda")
    mb.medusa_topk_tree_tokens(tree, head, k, root, idx, tok)
    torch.cuda.synchronize()
    vl = torch.from_numpy(st.verify_logits_for(c2, tree, idx.cpu().numpy(), root.cpu().numpy())).cuda()
    ur = np.random.default_rng(cfg.cfg_id * 7919)
    u_node = torch.from_numpy(ur.random((B, T)).astype(np.float32)).cuda()
    u_bonus = torch.from_numpy(ur.random(B).astype(np.float32)).cuda()
    out = {n: torch.empty(B, dtype=torch.int32, device="cuda") for n in ("len", "best", "next")}
    acc = torch.empty((B, tree.depth_max + 1), dtype=torch.int32, device="cuda")
    ws = mb.workspace(mb.typical_accept_workspace(tree, B, V))

    def typical(eps, tau):
        mb.typical_accept(tree, vl, tok, eps, cfg.delta, tau, out["len"], out["best"], out["next"], acc, ws=ws)

    def rejection(tau):
        mb.rejection_accept(tree, vl, head, tok, tau, u_node, u_bonus, out["len"], out["best"], out["next"], acc)

    def mean_len(fn):
        fn()
        return float(out["len"].float().mean().item())

    def time_us(fn, n=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    res = {"sweep": "accept", "workload": cfg.name, "sequences": B, "tree_nodes": T, "delta": cfg.delta,
           "eps_curve": [[e, mean_len(lambda: typical(e, 1.0))] for e in (0.01, 0.03, 0.05, 0.09, 0.15, 0.25)],
           "temperature_curve": {
               "typical": [[t, mean_len(lambda: typical(cfg.eps, t))] for t in (0.0, 0.25, 0.5, 0.7, 1.0, 1.5, 2.0)],
               "rejection": [[t, mean_len(lambda: rejection(t))] for t in (0.0, 0.25, 0.5, 0.7, 1.0, 1.5, 2.0)]},
           "us_per_call": {"typical": time_us(lambda: typical(cfg.eps, 1.0)),
                           "rejection": time_us(lambda: rejection(1.0))},
           "data": "synthetic: seeded head logits, verification logits planted at their top-k, seeded uniforms"}
    print(json.dumps(res), flush=True)


def device_info():
    import torch
    from speculative_decoding_05_amd import binding as mb
    p = torch.cuda.get_device_properties(0)
    cus, clock_khz, mem_khz = mb.device_info()
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": cus,
            "hbm_bytes": p.total_memory, "peak_clock_mhz": clock_khz / 1e3, "peak_memory_clock_mhz": mem_khz / 1e3}


def measured_peaks(read_bytes=4 << 30, reps=5):
    """The two roofs measured on this device in this run with the library's
    peak kernels: a read-only stream over read_bytes (16x the last-level
    cache), and a bf16 matrix-core loop of 4 independent 32x32x16 chains per
    wave on 2 blocks per CU, run for ~0.1 s first so the clock settles.  Best
    of `reps` timed calls each.  The matrix-core rate divided by the dense
    rate per clock (1024 flop per SIMD per clock) gives the clock the matrix
    cores would run at if they were busy every cycle."""
    import torch
    from speculative_decoding_05_amd import binding as mb
    buf = torch.ones(read_bytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda")

    def best_us(fn):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, 1e3 * e0.elapsed_time(e1))
        return best

    read_us = best_us(lambda: mb.peak_hbm_read(buf, sink))
    del buf
    torch.cuda.empty_cache()
    cus = mb.device_info()[0]
    blocks, iters = 2 * cus, 2000
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.1:
        mb.peak_mfma_bf16(blocks, iters, fsink)
        torch.cuda.synchronize()
    flops = mb.lib.medusa_peak_mfma_flops(blocks, iters)
    mfma_us = best_us(lambda: mb.peak_mfma_bf16(blocks, iters, fsink))
    mfma = flops / (mfma_us * 1e-6)
    return {"hbm_read_gbps": read_bytes / (read_us * 1e-6) / 1e9, "hbm_read_bytes": read_bytes,
            "mfma_bf16_tflops": mfma / 1e12, "mfma_implied_clock_ghz": mfma / (cus * 4 * 1024) / 1e9,
            "kernels": "medusa_peak_hbm_read, medusa_peak_mfma_bf16", "reps": reps}


def copy_rate(nbytes=1 << 30, reps=5):
    """Device-to-device copy of nbytes: (read + write bytes) / time, GB/s -- the
    measured counterpart of the 8 TB/s datasheet peak."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    rate = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return rate


def accept_histogram(s, depth_max):
    """Accepted candidates per sequence of the batch (synthetic planted
    verification logits; every rotated copy carries the same ones)."""
    counts = [0] * (depth_max + 1)
    s.run(0)
    for a in s.accept_len.cpu().tolist():
        counts[a] += 1
    return counts


def graph_variant(s, copies, steps, warmup):
    """The same step captured once per input copy in a HIP graph and replayed;
    every replay's outputs are compared with the eager step's on that copy."""
    import torch
    outs = lambda: [t.clone() for t in (s.tree_tok, s.attn, s.accept_len, s.best, s.next_tok, s.accepted)]
    eager = []
    for c in range(copies):
        s.run(c)
        eager.append(outs())
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm the launch paths off the capture
        s.run(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for c in range(copies):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            s.run(c)
        graphs.append(g)
    torch.cuda.synchronize()
    match = True
    for rep in range(2):               # replays with eager work and syncs between them
        for c in range(copies):
            graphs[c].replay()
            torch.cuda.synchronize()
            match &= all(torch.equal(a, b) for a, b in zip(outs(), eager[c]))
            s.run((c + 1) % copies)
            torch.cuda.synchronize()
    for i in range(warmup):
        graphs[i % copies].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        graphs[i % copies].replay()
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / steps
    return {"us_per_step": us, "steps_per_s": 1e6 / us, "replays_match_eager": bool(match)}


OTHER_WORKLOADS = ["tiny_f32", "roofline_b16", "vicuna13b_b8", "dense341_b32"]


def other_workload(name, steps, warmup, verify_reps=0):
    """Whole eager steps of another workload: inputs drawn on the device
    (same shapes and distributions as the headline's host-drawn ones),
    verification logits planted at the step's own candidates, per-step inputs
    rotated past the last-level cache; for bf16 workloads also the verify-pass
    contractions (`verify_reps` timed calls each).  No oracle."""
    import torch
    from speculative_decoding_05_amd import configs
    from speculative_decoding_05_amd import step as st
    cfg = configs.CONFIGS[name]
    tree = st.build_tree(cfg)
    e = elem(cfg)
    per_copy = (cfg.B * cfg.H * e + 3 * cfg.B * tree.T * cfg.nh * cfg.dh * e
                + 2 * cfg.B * cfg.nh * cfg.L * cfg.dh * e + cfg.B * tree.T * cfg.V * 4)
    copies = max(1, min(8, math.ceil(512 * 2 ** 20 / per_copy)))
    inp = st.device_inputs(cfg, tree.T, seed=cfg.cfg_id)
    s = st.Step(cfg, tree, inp, copies=copies)
    del inp
    torch.cuda.empty_cache()
    s.heads()
    s.heads_vocab()
    s.topk_and_tokens()
    torch.cuda.synchronize()
    s.set_verify_logits(st.verify_logits_for(cfg, tree, s.topk_idx.cpu().numpy(), s.root.cpu().numpy()))
    us, stage = time_steps(s, steps, warmup, copies)
    sb, sf = stage_bytes(cfg, tree), stage_flops(cfg, tree)
    names = list(stage)
    roof_s = sum(max(sb[n] / HBM_PEAK, sf.get(n, 0) / flop_peak(cfg)) for n in names)
    out = {"tree_steps_per_s": 1e6 / us, "seq_steps_per_s": cfg.B * 1e6 / us, "us_per_step": us,
           "steps": steps, "input_copies": copies, "step_roofline_us": roof_s * 1e6,
           "hbm_roofline_frac_step": roof_s / (us * 1e-6), "stage_us": stage,
           "stage_gbps": {n: sb[n] / (stage[n] * 1e-6) / 1e9 for n in names},
           "config": {"batch": cfg.B, "hidden": cfg.H, "attn_heads": cfg.nh, "kv_len": cfg.L,
                      "medusa_heads": cfg.K, "tree_nodes": tree.T, "topk": cfg.k},
           "data": "synthetic, drawn on the device (torch generator); planted verification logits"}
    if name == "roofline_b16":
        out["verify_step"] = composed_step(s, steps, warmup, copies, seed=cfg.cfg_id)
    if cfg.dtype == "bf16" and verify_reps > 0:
        out["verify_pass"] = verify_pass(s, verify_reps)
    del s
    torch.cuda.empty_cache()
    return out


def copy_probe(nbytes):
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "launches": 3}), flush=True)


def cpu_baseline(cfg, host, budget_s):
    """The oracle, as it stands, on whole steps of the same workload."""
    import numpy as np
    import oracle
    from speculative_decoding_05_amd import configs, synth
    from speculative_decoding_05_amd import step as st

    f = synth.as_f64
    spec = cfg.tree
    paths = (oracle.dense_paths(cfg.K, spec.k) if spec.kind == "dense"
             else oracle.greedy_paths(configs.acc_exact, cfg.K, spec.n_paths, spec.rank_cap))
    ot = oracle.build_tree(paths, cfg.K, spec.k)
    args = {n: f(host[n]) for n in ("h", "W1", "W2", "q", "kt", "vt", "kc", "vc")}
    rnd = cfg.dtype == "bf16"
    # the verification logits are planted at the oracle's own candidates (setup, untimed)
    idx, _ = oracle.topk_per_head(oracle.medusa_heads(args["h"], args["W1"], args["W2"], rnd), cfg.k)
    vl = synth.verification_logits(cfg.cfg_id, cfg.V, ot["parent"], ot["depth"], ot["rank"], idx,
                                   host["root_tok"], configs.acc_float, cfg.k).astype(np.float64)
    n, t0 = 0, time.perf_counter()
    while True:
        last = oracle.step(args["h"], args["W1"], args["W2"], host["root_tok"], ot, cfg.k, args["q"], args["kt"],
                           args["vt"], args["kc"], args["vc"], vl, cfg.eps, cfg.delta, cfg.temperature,
                           round_r_bf16=rnd)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 100:
            break
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        cores = 1
    return {"value": n / el, "unit": "tree-steps/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} whole steps of {cfg.name} (B={cfg.B}) in float64 NumPy; "
                      f"BLAS threads={cores}, host cpus={len(os.sched_getaffinity(0))}"}, last, vl, ot


def step_parity(s, last, vl, ot):
    """The GPU step on input copy 0 against the oracle step just timed (same
    seeded inputs; the verification logits are planted at the oracle's
    candidates and given to both): tree tokens bit-exact, and acceptance under
    the flag rule (a decision within 1e-3 of its threshold may go either way;
    every other decision, and the outputs as the scan of the GPU's own
    decisions, must match)."""
    import numpy as np
    import torch
    from speculative_decoding_05_amd import binding as mb
    cfg = s.cfg
    B, T = cfg.B, ot["T"]
    s.heads(0)
    s.heads_vocab(0)
    s.topk_and_tokens(0)
    torch.cuda.synchronize()
    tok_g = s.tree_tok.cpu().numpy().astype(np.int64)
    tok_o = last["tree_tok"]
    cp = torch.empty((B, T), dtype=torch.float32, device="cuda")
    th = torch.empty((B, T), dtype=torch.float32, device="cuda")
    vld = torch.from_numpy(vl.astype(np.float32)).cuda()
    tokd = torch.from_numpy(tok_o.astype(np.int32)).cuda()
    mb.typical_accept(s.tree, vld, tokd, cfg.eps, cfg.delta, cfg.temperature, s.accept_len, s.best, s.next_tok,
                      s.accepted, cp, th, s.ws_acc)
    torch.cuda.synchronize()
    ref = last["accept"]
    p_g, thr_g = cp.cpu().numpy(), th.cpu().numpy()
    alen, best, nxt = s.accept_len.cpu().numpy(), s.best.cpu().numpy(), s.next_tok.cpu().numpy()
    flagged = mismatches = 0
    for b in range(B):
        dec = np.zeros(T, bool)
        acc = np.zeros(T, bool)
        acc[0] = True
        bad = False
        for c in range(1, T):
            n = ot["parent"][c]
            dec[c] = p_g[b, c] > thr_g[b, n]
            acc[c] = acc[n] and dec[c]
            if abs(ref["p"][b, c] - ref["thr"][b, c]) < 1e-3:
                flagged += 1
            elif dec[c] != ref["dec"][b, c]:
                bad = True
        a = int(ot["depth"][acc].max())
        bst = int(np.flatnonzero(acc & (ot["depth"] == a))[0])
        bad |= alen[b] != a or best[b] != bst or nxt[b] != int(np.argmax(vl[b, bst]))
        mismatches += int(bad)
    return {"sequences": B, "tree_tokens_equal": bool(np.array_equal(tok_g, tok_o)),
            "decisions": B * (T - 1), "flagged_decisions": flagged, "mismatched_sequences": mismatches,
            "accept_len_gpu": alen.tolist(), "accept_len_oracle": ref["accept_len"].tolist()}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", default="vicuna7b_b1")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget (0: skip)")
    ap.add_argument("--rotate-mb", type=float, default=512.0, help="bytes of rotated per-step inputs")
    ap.add_argument("--copy-probe", type=int, default=0, help="only copy this many bytes (counter calibration)")
    ap.add_argument("--sweep", choices=["trees", "accept"], default=None,
                    help="instead of the headline line: step time per tree size, or acceptance curves")
    ap.add_argument("--graph", type=int, default=1, help="also time the step captured in HIP graphs (0: skip)")
    ap.add_argument("--composed", type=int, default=100,
                    help="steps of the verify step with LM-head verification logits (0: skip)")
    ap.add_argument("--verify-reps", type=int, default=10,
                    help="repetitions of each verify-pass contraction (0: skip)")
    ap.add_argument("--event-every", type=int, default=8,
                    help="bracket the vocabulary projection with events on every n-th timed step")
    ap.add_argument("--others", type=int, default=1,
                    help="also time eager steps of the other bf16 workloads (0: skip)")
    ap.add_argument("--peaks", type=int, default=1, help="measure the HBM-read and bf16 matrix-core peaks (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: only one GPU is measured; the verify tree-step has no "
              "multi-GPU path (sequences would shard across GPUs with no exchange).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from speculative_decoding_05_amd import build as b
    if not os.path.exists(b.LIB):
        b.build()
    if args.copy_probe:
        copy_probe(args.copy_probe)
        return
    if args.sweep:
        from speculative_decoding_05_amd import configs as _c
        torch.cuda.set_device(0)
        cfg = _c.CONFIGS[args.config]
        (tree_sweep if args.sweep == "trees" else accept_sweep)(cfg, args)
        return
    from speculative_decoding_05_amd import configs
    from speculative_decoding_05_amd import step as st

    cfg = configs.CONFIGS[args.config]
    torch.cuda.set_device(0)
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    tree = st.build_tree(cfg)
    host = st.host_inputs(cfg, tree.T)
    e = elem(cfg)
    per_copy = (cfg.B * cfg.H * e + 3 * cfg.B * tree.T * cfg.nh * cfg.dh * e
                + 2 * cfg.B * cfg.nh * cfg.L * cfg.dh * e + cfg.B * tree.T * cfg.V * 4)
    copies = max(1, min(64, math.ceil(args.rotate_mb * 2 ** 20 / per_copy)))
    s = st.Step(cfg, tree, host, copies=copies)
    # candidates of this step's heads, then the planted verification logits
    s.heads()
    s.heads_vocab()
    s.topk_and_tokens()
    torch.cuda.synchronize()
    vl = st.verify_logits_for(cfg, tree, s.topk_idx.cpu().numpy(), host["root_tok"])
    s.set_verify_logits(vl)
    print(f"[bench] {cfg.name}: {copies} input copies, warmup {args.warmup}, timing {args.steps}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        s.run(i % copies)
    torch.cuda.synchronize()
    ev_steps = list(range(0, args.steps, max(1, args.event_every)))
    ev = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in ev_steps}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    # ten equal sub-intervals of the timed steps (median / best reporting)
    n_rep = 10 if args.steps >= 10 else 1
    rep_at = {round(r * args.steps / n_rep): torch.cuda.Event(enable_timing=True) for r in range(1, n_rep)}
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        if i in rep_at:
            rep_at[i].record()
        c = i % copies
        s.heads(c)
        if i in ev:
            ev[i][0].record()
        s.heads_vocab(c)
        if i in ev:
            ev[i][1].record()
        s.topk_and_tokens(c)
        s.attention(c)
        s.accept(c)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t_start.elapsed_time(t_end)
    ms_step = ms / args.steps
    marks = [(0, t_start)] + sorted(rep_at.items()) + [(args.steps, t_end)]
    rep_rates = sorted((b - a) / (ea.elapsed_time(eb) * 1e-3) for (a, ea), (b, eb) in zip(marks, marks[1:]))
    vocab_ms = sum(a.elapsed_time(bb) for a, bb in ev.values()) / len(ev)

    # per-stage times from a separate instrumented pass (not the timed region)
    names = ["head_resblock", "head_vocab", "topk_tokens", "attention", "accept"]
    fns = [s.heads, s.heads_vocab, s.topk_and_tokens, s.attention, s.accept]
    n_inst = min(100, args.steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(n_inst)]
    for i in range(n_inst):
        evs[i][0].record()
        for j, fn in enumerate(fns):
            fn(i % copies)
            evs[i][j + 1].record()
    torch.cuda.synchronize()
    stage_us = {n: 1e3 * sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(n_inst)) / n_inst
                for j, n in enumerate(names)}

    sb = stage_bytes(cfg, tree)
    sf = stage_flops(cfg, tree)
    roof_s = sum(max(sb[n] / HBM_PEAK, sf.get(n, 0) / flop_peak(cfg)) for n in names)
    vocab_bytes = sb["head_vocab"]
    achieved = vocab_bytes / (vocab_ms * 1e-3)
    res = {
        "metric": METRIC,
        "value": args.steps / (ms * 1e-3),
        "unit": "tree-steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) activations/cache, N(0,0.02) weights, planted verification logits)",
        "config": {"workload": cfg.name, "batch": cfg.B, "hidden": cfg.H, "attn_heads": cfg.nh,
                   "head_dim": cfg.dh, "vocab": cfg.V, "kv_len": cfg.L, "medusa_heads": cfg.K,
                   "tree_nodes": tree.T, "topk": cfg.k, "eps": cfg.eps, "delta": cfg.delta,
                   "parallelism": "single GPU"},
        "seq_steps_per_s": cfg.B * args.steps / (ms * 1e-3),
        "hbm_roofline_frac_step": roof_s / (ms_step * 1e-3),
        "step_roofline_us": roof_s * 1e6,
        "stage_us": stage_us,
        "wall_s_timed": wall,
        "input_copies": copies,
        "roofline": {"bound": "hbm", "kernel": "head_gemm_bf16 (vocabulary projection W2)",
                     "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK, "traffic": counted_traffic(cfg.name),
                     "bytes_per_launch": vocab_bytes, "avg_launch_us": vocab_ms * 1e3,
                     "launches_timed": len(ev)},
    }
    res["steps_per_s_median"] = rep_rates[len(rep_rates) // 2]
    res["steps_per_s_best"] = rep_rates[-1]
    res["stage_gbps"] = {n: sb[n] / (stage_us[n] * 1e-6) / 1e9 for n in names}
    res["device"] = device_info()
    res["hbm_copy_gbps"] = copy_rate()   # device-to-device copy, read + write bytes
    if args.peaks:
        print("[bench] measured peaks", file=sys.stderr, flush=True)
        pk = measured_peaks()
        res["measured_peaks"] = pk
        hbm_m, mfma_m = pk["hbm_read_gbps"] * 1e9, pk["mfma_bf16_tflops"] * 1e12
        res["roofline"]["peak_measured"] = pk["hbm_read_gbps"]
        res["roofline"]["frac_measured"] = achieved / hbm_m
        roof_m = sum(max(sb[n] / hbm_m, sf.get(n, 0) / mfma_m) for n in names)
        res["step_roofline_us_measured_peaks"] = roof_m * 1e6
        res["hbm_roofline_frac_step_measured_peaks"] = roof_m / (ms_step * 1e-3)
    res["accept_len_histogram"] = accept_histogram(s, tree.depth_max)
    if args.graph:
        res["hip_graph"] = graph_variant(s, copies, args.steps, args.warmup)
    if cfg.dtype == "bf16" and args.verify_reps > 0:
        print("[bench] verify-pass contractions (M = B*T rows)", file=sys.stderr, flush=True)
        res["verify_pass"] = verify_pass(s, args.verify_reps)
    if cfg.dtype == "bf16" and args.composed > 0:
        print("[bench] verify step with computed verification logits", file=sys.stderr, flush=True)
        res["verify_step"] = composed_step(s, args.composed, 10, copies, seed=cfg.cfg_id)
    print(f"[bench] {ms_step * 1e3:.1f} us/step; stages {json.dumps({k: round(v, 1) for k, v in stage_us.items()})}",
          file=sys.stderr, flush=True)
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"], last, vl_o, ot = cpu_baseline(cfg, host, args.cpu_seconds)
        res["parity_vs_oracle"] = step_parity(s, last, vl_o, ot)
    else:
        res["cpu_baseline"] = None
    if args.others and cfg.name == "vicuna7b_b1":
        del s
        torch.cuda.empty_cache()
        res["other_workloads"] = {}
        for name in OTHER_WORKLOADS:
            print(f"[bench] other workload {name}", file=sys.stderr, flush=True)
            n = 40 if name == "dense341_b32" else 100
            res["other_workloads"][name] = other_workload(name, n, 10, args.verify_reps)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()

"""Seeded synthetic inputs for the verify tree-step.

Shared by the HIP path's tests and bench and by the CPU oracle's tests.
Holds none of the method's arithmetic: it only draws numbers, rounds them
to the storage type, and plants synthetic verification logits at token ids
it is given.

Streams: numpy Generator(PCG64(SeedSequence([cfg_id, role, b]))); b is
the sequence index, or SHARED for tensors common to the batch (weights).
Normals are drawn as float32, scaled, and for bf16 storage rounded to
nearest-even on the fp32 bit pattern.  bf16 tensors are returned as
uint16 bit patterns, fp32 tensors as float32.
"""
from __future__ import annotations

import math

import numpy as np

SHARED = 2 ** 32 - 1
ROLE_W1, ROLE_W2, ROLE_H, ROLE_ROOT = 1, 2, 3, 4
ROLE_Q, ROLE_KT, ROLE_VT, ROLE_KC, ROLE_VC, ROLE_VLOGITS = 5, 6, 7, 8, 9, 10
ROLE_NODE_H, ROLE_W_LM = 11, 12
WEIGHT_STD = 0.02


def rng(cfg_id: int, role: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg_id, role, b])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 view of a stored tensor (bf16 bits or float32)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(x32) if dtype == "bf16" else x32


def normal(cfg_id, role, b, shape, std, dtype, chunks=1):
    """N(0, std^2) tensor of `shape`; drawn in `chunks` equal slices of the
    leading axis from one stream (same values for any chunking)."""
    g = rng(cfg_id, role, b)
    out = np.empty(shape, dtype=np.uint16 if dtype == "bf16" else np.float32)
    n0 = shape[0]
    step = max(1, -(-n0 // chunks))
    for s in range(0, n0, step):
        e = min(n0, s + step)
        x = g.standard_normal((e - s,) + tuple(shape[1:]), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[s:e] = _store(x, dtype)
    return out


def per_sequence(cfg_id, role, B, shape, std, dtype):
    """[B] + shape, sequence b drawn from its own stream."""
    out = np.empty((B,) + tuple(shape), dtype=np.uint16 if dtype == "bf16" else np.float32)
    for b in range(B):
        x = rng(cfg_id, role, b).standard_normal(tuple(shape), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out[b] = _store(x, dtype)
    return out


# --- the tensors of one configuration -------------------------------------------
def head_weights(cfg):
    """W1 [K][H][H] and W2 [K][V][H], N(0, 0.02^2), shared by the batch."""
    W1 = normal(cfg.cfg_id, ROLE_W1, SHARED, (cfg.K, cfg.H, cfg.H), WEIGHT_STD, cfg.dtype, chunks=cfg.K)
    W2 = normal(cfg.cfg_id, ROLE_W2, SHARED, (cfg.K, cfg.V, cfg.H), WEIGHT_STD, cfg.dtype, chunks=cfg.K * 4)
    return W1, W2


def node_hidden(cfg, M):
    """Hidden states of M tree nodes [M][H] ~ N(0, 1) (the verify-pass rows)."""
    return normal(cfg.cfg_id, ROLE_NODE_H, SHARED, (M, cfg.H), 1.0, cfg.dtype, chunks=max(1, M // 1024))


def lm_head_weights(cfg):
    """The backbone's LM head W_lm [V][H] ~ N(0, 0.02^2)."""
    return normal(cfg.cfg_id, ROLE_W_LM, SHARED, (cfg.V, cfg.H), WEIGHT_STD, cfg.dtype, chunks=8)


def hidden(cfg, B=None):
    """Last hidden state h [B][H] ~ N(0, 1)."""
    return per_sequence(cfg.cfg_id, ROLE_H, cfg.B if B is None else B, (cfg.H,), 1.0, cfg.dtype)


def root_tokens(cfg, B=None):
    B = cfg.B if B is None else B
    return np.array([rng(cfg.cfg_id, ROLE_ROOT, b).integers(cfg.V) for b in range(B)], dtype=np.int32)


def tree_qkv(cfg, T, B=None):
    """Query, key and value of every tree token, [B][T][nh][dh] ~ N(0, 1)."""
    B = cfg.B if B is None else B
    shape = (T, cfg.nh, cfg.dh)
    return tuple(per_sequence(cfg.cfg_id, role, B, shape, 1.0, cfg.dtype)
                 for role in (ROLE_Q, ROLE_KT, ROLE_VT))


def kv_cache(cfg, B=None, L=None):
    """Prefix cache K and V, [B][nh][L][dh] ~ N(0, 1)."""
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    shape = (cfg.nh, L, cfg.dh)
    return tuple(per_sequence(cfg.cfg_id, role, B, shape, 1.0, cfg.dtype)
                 for role in (ROLE_KC, ROLE_VC))


def verification_logits(cfg_id, V, parent, depth, rank, topk_idx, root_tok, acc, k):
    """Synthetic verification logits [B][T][V] float32.

    They stand in for what the backbone would output at every tree node.
    Per sequence b (own stream) and node n in order:
      * background: log-probabilities of N(0,1) scores with total mass
        r ~ U(0.02, 0.2);
      * if n has children (depth d): a planted rank i* = first i < k with
        U_i < acc(d, i) (maybe none), token t1 = topk_idx[d][b][i*] with
        probability p1 = (1 - r) U(0.5, 1); a second token t2, one of n's
        children other than rank i*, with probability
        p2 = min(exp(U(ln 1e-4, ln 0.3)), 0.9 (1 - r - p1));
      * a distractor token t3 (not the root token, t1, t2, nor any child of
        n) takes the remaining mass max(1 - r - p1 - p2, 1e-12), when the
        vocabulary holds such a token;
      * finally a row offset U(-5, 5).
    parent/depth/rank: node arrays of the tree; topk_idx [K][B][k];
    root_tok [B]; acc(d, i) -> float.
    """
    parent = np.asarray(parent)
    depth = np.asarray(depth)
    rank = np.asarray(rank)
    topk_idx = np.asarray(topk_idx)
    T = parent.shape[0]
    B = topk_idx.shape[1]
    K = topk_idx.shape[0]
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[int(parent[c])].append(c)
    out = np.empty((B, T, V), dtype=np.float32)
    lo, hi = math.log(1e-4), math.log(0.3)
    for b in range(B):
        g = rng(cfg_id, ROLE_VLOGITS, b)
        for n in range(T):
            r = g.uniform(0.02, 0.2)
            z = g.standard_normal(V)
            m = z.max()
            z = z - (m + math.log(np.exp(z - m).sum())) + math.log(r)
            kids = children[n]
            planted = []
            p1 = p2 = 0.0
            excl = {int(root_tok[b])}
            if kids:
                d = int(depth[n])
                u = g.uniform(size=k)
                istar = next((i for i in range(k) if u[i] < acc(d, i)), None)
                p1_draw = (1.0 - r) * g.uniform(0.5, 1.0)
                kid_tok = [int(topk_idx[d, b, rank[c]]) for c in kids] if d < K else []
                excl.update(kid_tok)
                if istar is not None and d < K:
                    p1 = p1_draw
                    t1 = int(topk_idx[d, b, istar])
                    planted.append((t1, p1))
                    excl.add(t1)
                others = [int(rank[c]) for c in kids if int(rank[c]) != istar]
                if others and d < K:
                    j = others[int(g.integers(len(others)))]
                    p2 = min(math.exp(g.uniform(lo, hi)), 0.9 * (1.0 - r - p1))
                    t2 = int(topk_idx[d, b, j])
                    planted.append((t2, p2))
                    excl.add(t2)
            if len(excl) < V:   # a vocabulary this small may have no token left for it
                while True:
                    t3 = int(g.integers(V))
                    if t3 not in excl:
                        break
                p3 = max(1.0 - r - p1 - p2, 1e-12)
                planted.append((t3, p3))
            for t, p in planted:
                z[t] = math.log(p)
            z += g.uniform(-5.0, 5.0)
            out[b, n] = z.astype(np.float32)
    return out

"""Plain CPU oracle for one Medusa verify tree-step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module: only the test-suite, the smoke check and the bench's
CPU-baseline leg do.  It shares no code, table or helper with the HIP
library; both sides only consume the same seeded inputs.

Every function is the method's plain definition, evaluated in float64
(inputs are exact: bf16 and fp32 values convert to float64 without loss),
one step after the other, with library matmuls as the only primitive.

Sources (pages as published):
  [P3]  "Medusa: Simple LLM Inference Acceleration Framework with Multiple
        Decoding Heads" -- ICML 2024 paper summary (mhpq.cn).  Sections:
        "基准/方法设计" (the three components: heads, tree attention,
        typical acceptance), "方法细节" (sparse-tree construction,
        temperature), FAQ "树注意力为什么能一次验证多条候选".
  [P2]  "Medusa 多解码头推理加速全解析" (bjdmk.com.cn).  Sections
        "核心架构" (tree example), "推理算法" (candidate generation,
        tree verification), "超参数调优指南" (per-head top-k,
        medusa_choices), "部署与生成" (generate arguments).

Readings of points the pages leave open are listed per function.
Parity pins: every function here is pinned by tests under tests/ against
closed forms, brute force or library routines (see the test module names
test_oracle_*).
"""
from __future__ import annotations

import heapq
import itertools
import math
from fractions import Fraction

import numpy as np


class TreeError(ValueError):
    """A path list that does not describe a valid candidate tree."""


# ----------------------------------------------------------------------------
# rounding point
# ----------------------------------------------------------------------------
def bf16_round(x):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits.  With x = m * 2**e, 0.5 <= |m| < 1,
    the nearest value is rint(m * 2**8) / 2**8 * 2**e (np.rint rounds half
    to even).  Used only where the HIP path stores an intermediate in bf16
    (the head ResBlock output feeding the vocabulary projection).
    Valid for values in the bf16 normal range; inf and nan pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    out = np.ldexp(np.rint(m * 256.0) / 256.0, e)
    return np.where(np.isfinite(x), out, x)


# ----------------------------------------------------------------------------
# (1) Medusa heads  -- [P3] "基准/方法设计", first component
# ----------------------------------------------------------------------------
def medusa_heads(h, W1, W2, round_r_bf16=False):
    """Logits of the K Medusa heads on rows h.

    Head k (predicting token t+k+1) computes
        p^(k) = softmax(W2^(k) (SiLU(W1^(k) h) + h)),
    [P3] "基准/方法设计" (the extraction drops '=' and '+'; the residual
    reading is the only one consistent with the stated initialisation:
    W1 = 0 must reproduce the backbone's prediction).  The softmax is left
    to the consumer, so this returns the pre-softmax logits.

    h  [M][H], W1 [K][H][H] (row = output feature), W2 [K][V][H].
    Readings: no bias terms; SiLU(x) = x * sigmoid(x); in the bf16
    configuration the ResBlock output r is stored as bf16 before the
    vocabulary projection (round_r_bf16=True).
    Returns float64 logits [K][M][V].
    """
    h = np.asarray(h, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    K = W1.shape[0]
    M = h.shape[0]
    V = W2.shape[1]
    logits = np.empty((K, M, V), dtype=np.float64)
    for k in range(K):
        u = h @ W1[k].T                       # u[m][o] = sum_i W1[k][o][i] h[m][i]
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-u))
        r = h + u * sig
        if round_r_bf16:
            r = bf16_round(r)
        logits[k] = r @ W2[k].T               # logits[m][n] = sum_i W2[k][n][i] r[m][i]
    return logits


def verification_logits(x, W_lm):
    """The backbone's logits at every tree node: its LM head applied to the
    node's hidden state.  [P3] "基准/方法设计" gives the LM head as the W1 = 0
    case of the head formula (SiLU(0) = 0, so r = h), i.e. a plain projection
        z[b][t][v] = sum_i W_lm[v][i] x[b][t][i].
    x [B][T][H], W_lm [V][H].  Reading: the hidden state handed to the LM head
    is whatever the caller supplies (here, the tree-attention output of the
    node with heads concatenated); the backbone layers between attention and
    the LM head are outside this path.  Returns float64 [B][T][V].
    """
    x = np.asarray(x, dtype=np.float64)
    W_lm = np.asarray(W_lm, dtype=np.float64)
    B, T, H = x.shape
    return (x.reshape(B * T, H) @ W_lm.T).reshape(B, T, W_lm.shape[0])


# ----------------------------------------------------------------------------
# (2) per-head top-k  -- [P2] "推理算法 / 候选生成", "超参数调优指南 / 每头 Top-K"
# ----------------------------------------------------------------------------
def medusa_topk(logits, k):
    """Top-k of each row, ordered by (value descending, index ascending).

    The pages take torch.topk of each head's logits; they say nothing of
    ties.  Reading: equal values go to the lower token id, which makes the
    answer unique.  -0.0 and +0.0 compare equal.
    logits [R][V] -> (idx [R][k] int64, val [R][k] float64).
    """
    logits = np.asarray(logits, dtype=np.float64)
    R, V = logits.shape
    if not (1 <= k <= V):
        raise ValueError("k must be in [1, V]")
    idx = np.empty((R, k), dtype=np.int64)
    val = np.empty((R, k), dtype=np.float64)
    cols = np.arange(V)
    for r in range(R):
        order = np.lexsort((cols, -logits[r]))[:k]  # primary key -value, then index
        idx[r] = order
        val[r] = logits[r, order]
    return idx, val


# ----------------------------------------------------------------------------
# candidate trees  -- [P2] "核心架构", "推理算法", "树结构：medusa_choices";
#                     [P3] "方法细节" (sparse tree)
# ----------------------------------------------------------------------------
def dense_paths(K, k):
    """All rank paths of a dense tree: every combination of the per-head
    top-k, depth 1..K ([P2] "候选生成": Cartesian product of the heads'
    top-k lists; with intermediate nodes kept so that every prefix is a
    node of the tree)."""
    out = []
    for d in range(1, K + 1):
        out.extend(tuple(p) for p in itertools.product(range(k), repeat=d))
    return out


def greedy_paths(acc, K, n_paths, rank_cap):
    """Sparse tree built greedily from per-head top-i accuracies.

    [P3] "方法细节": estimate each head's top-i accuracy, then repeatedly
    add the node with the largest expected gain in accept length.  Under
    the pages' independence model a node's gain is the probability that
    its whole rank path is right: prod_d acc(d, i_d).  The frontier holds
    the children (ranks < rank_cap, depth <= K) of nodes already in the
    tree; the root is always present.

    acc(d, i) must return exact numbers (Fraction) so that equal products
    compare equal.  Reading for equal gains: shorter path first, then the
    lexicographically smaller path.
    Returns the chosen paths in the order they were added.
    """
    heap = []

    def push(path, score):
        heapq.heappush(heap, (-score, len(path), path))

    for i in range(rank_cap):
        push((i,), Fraction(acc(0, i)))
    chosen = []
    while len(chosen) < n_paths:
        if not heap:
            raise TreeError("not enough candidate paths")
        neg, _, path = heapq.heappop(heap)
        chosen.append(path)
        if len(path) < K:
            for i in range(rank_cap):
                push(path + (i,), -neg * Fraction(acc(len(path), i)))
    return chosen


def validate_paths(paths, K, k):
    """Reject path lists that do not describe a tree ([P2] medusa_choices:
    each entry is a path of per-head rank choices, and a path is only
    meaningful if every shorter prefix is also a node)."""
    seen = set()
    for p in paths:
        p = tuple(int(x) for x in p)
        if not (1 <= len(p) <= K):
            raise TreeError(f"path {p}: length outside [1, {K}]")
        if any(r < 0 or r >= k for r in p):
            raise TreeError(f"path {p}: rank outside [0, {k})")
        if p in seen:
            raise TreeError(f"path {p}: duplicate")
        seen.add(p)
    for p in seen:
        for n in range(1, len(p)):
            if p[:n] not in seen:
                raise TreeError(f"path {p}: prefix {p[:n]} missing")


def build_tree(paths, K, k):
    """Node arrays of the candidate tree.

    Node 0 is the root (the greedily chosen next token, [P3]
    "基准/方法设计": the first token is taken greedily); node j >= 1 is the
    j-th path in (length, lexicographic) order -- reading: the pages fix no
    order; this one puts every parent before its children.
    parent(j) = node of path[:-1]; depth(j) = len(path); rank(j) = last
    element; head(j) = depth - 1 (0-based Medusa head, head 0 predicts the
    token after the root).
    mask: bit i of row j set iff path_i is a prefix of path_j (root and j
    itself included) -- [P3] each token sees only the predecessors on its
    own branch.
    retrieve: one row per leaf (leaves in node order), node ids root..leaf,
    padded with -1 to depth_max+1.
    """
    validate_paths(paths, K, k)
    nodes = [()] + sorted((tuple(int(x) for x in p) for p in paths),
                          key=lambda p: (len(p), p))
    index = {p: i for i, p in enumerate(nodes)}
    T = len(nodes)
    W = (T + 63) // 64
    parent = np.full(T, -1, dtype=np.int64)
    depth = np.zeros(T, dtype=np.int64)
    rank = np.full(T, -1, dtype=np.int64)
    head = np.full(T, -1, dtype=np.int64)
    for j in range(1, T):
        p = nodes[j]
        parent[j] = index[p[:-1]]
        depth[j] = len(p)
        rank[j] = p[-1]
        head[j] = len(p) - 1
    mask = np.zeros((T, W), dtype=np.uint64)
    for j in range(T):
        pj = nodes[j]
        for i in range(T):
            pi = nodes[i]
            if len(pi) <= len(pj) and pj[:len(pi)] == pi:
                mask[j, i // 64] |= np.uint64(1) << np.uint64(i % 64)
    has_child = np.zeros(T, dtype=bool)
    has_child[parent[1:]] = True
    leaves = [j for j in range(T) if not has_child[j]]
    depth_max = int(depth.max())
    retrieve = np.full((len(leaves), depth_max + 1), -1, dtype=np.int64)
    for r, leaf in enumerate(leaves):
        chain = []
        j = leaf
        while j != -1:
            chain.append(j)
            j = parent[j]
        chain.reverse()
        retrieve[r, :len(chain)] = chain
    return {
        "paths": nodes[1:], "T": T, "W": W, "K": K, "k": k,
        "parent": parent, "depth": depth, "rank": rank, "head": head,
        "mask": mask, "retrieve": retrieve, "n_leaves": len(leaves),
        "depth_max": depth_max,
    }


def ancestors(tree, j):
    """anc*(j): j, its parent, ..., the root, returned in increasing node order."""
    out = []
    while j != -1:
        out.append(int(j))
        j = tree["parent"][j]
    return sorted(out)


def tree_positions(tree, L):
    """Position of each tree token: prefix length + depth.  [P3] FAQ: the
    position encoding follows the tree (reading: a node at depth d sits d
    places after the last prefix token)."""
    return L + tree["depth"].copy()


def tree_tokens(tree, root_tok, topk_idx):
    """Token of every tree node per sequence.

    root_tok [B]; topk_idx [K][B][k].  Node 0 holds the root token, node j
    the rank(j)-th candidate of Medusa head head(j)  ([P2] "候选生成":
    the candidate is the base token followed by one choice per head).
    Returns [B][T] int64.
    """
    root_tok = np.asarray(root_tok)
    topk_idx = np.asarray(topk_idx)
    B = root_tok.shape[0]
    T = tree["T"]
    out = np.empty((B, T), dtype=np.int64)
    for b in range(B):
        out[b, 0] = root_tok[b]
        for j in range(1, T):
            out[b, j] = topk_idx[tree["head"][j], b, tree["rank"][j]]
    return out


# ----------------------------------------------------------------------------
# (3) tree attention  -- [P3] "基准/方法设计" second component, FAQ
# ----------------------------------------------------------------------------
def tree_attention(q, k_tree, v_tree, k_cache, v_cache, tree, scale=None, sel=None):
    """Attention of every tree node over the prefix cache plus its own ancestors.

    For sequence b, head h and node j:
        keys   = [K_cache[b,h,0:L] ; K_tree[b, i, h] for i in anc*(j)]
        values = [V_cache[b,h,0:L] ; V_tree[b, i, h] for i in anc*(j)]
        o      = softmax(keys . q[b,j,h] * scale) . values
    [P3]: candidates share the prefix; each token attends only to the
    predecessors on its own branch (plus itself, as in causal attention).
    scale defaults to 1/sqrt(dh) (reading; the pages do not state it).
    q, k_tree, v_tree [B][T][nh][dh]; k_cache, v_cache [B][nh][L][dh].
    sel: optional iterable of (b, h) pairs to evaluate (others stay nan),
    so that large shapes can be sampled.
    Returns float64 [B][T][nh][dh].
    """
    q = np.asarray(q, dtype=np.float64)
    k_tree = np.asarray(k_tree, dtype=np.float64)
    v_tree = np.asarray(v_tree, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    B, T, nh, dh = q.shape
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(dh)
    out = np.full((B, T, nh, dh), np.nan)
    pairs = [(b, h) for b in range(B) for h in range(nh)] if sel is None else list(sel)
    anc = [ancestors(tree, j) for j in range(T)]
    for b, h in pairs:
        for j in range(T):
            keys = np.concatenate([k_cache[b, h], k_tree[b, anc[j], h]], axis=0)
            vals = np.concatenate([v_cache[b, h], v_tree[b, anc[j], h]], axis=0)
            s = keys @ q[b, j, h] * scale
            w = np.exp(s - s.max())
            out[b, j, h] = (w / w.sum()) @ vals
    return out


# ----------------------------------------------------------------------------
# (4) typical acceptance  -- [P3] "基准/方法设计" third component; "方法细节"
# ----------------------------------------------------------------------------
def row_distribution(z, temperature):
    """softmax(z / temperature) of one row, its entropy (natural log,
    0 ln 0 = 0) and its argmax (lowest index).  temperature 0 is the
    greedy limit: a one-hot distribution at the argmax ([P3] "方法细节":
    temperature 0 reduces to greedy decoding)."""
    z = np.asarray(z, dtype=np.float64)
    amax = int(np.argmax(z))
    if temperature == 0:
        P = np.zeros_like(z)
        P[amax] = 1.0
    else:
        y = z / temperature
        w = np.exp(y - y.max())
        P = w / w.sum()
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(P > 0, P * np.log(np.where(P > 0, P, 1.0)), 0.0)
    H = -terms.sum()
    return P, H, amax


def typical_accept(logits, tree_tok, tree, eps, delta, temperature=1.0):
    """Typical acceptance over the candidate tree, per sequence.

    [P3] "基准/方法设计": a candidate x is kept if
        p(x) > min(eps, delta * exp(-H(p))),
    the first token is accepted greedily and unconditionally, and the
    longest accepted prefix goes on to the next step.
    Readings: p is the verification distribution at x's parent node (the
    one forward pass yields a distribution at every node); H uses the
    natural log; a node is accepted only if its parent is; among accepted
    nodes of greatest depth the smallest node index wins; the next greedy
    token is the argmax (lowest index) of the winner's row.

    logits [B][T][V]; tree_tok [B][T].
    Returns a dict: accept_len [B], best [B], next_tok [B],
    accepted_tok [B][depth_max+1] (-1 padded), and per decision
    p [B][T] / thr [B][T] (the candidate's probability under its parent,
    and the parent's threshold; nan for the root), dec [B][T], acc [B][T].
    """
    logits = np.asarray(logits, dtype=np.float64)
    tree_tok = np.asarray(tree_tok)
    B, T, V = logits.shape
    parent, depth = tree["parent"], tree["depth"]
    Dm = tree["depth_max"]
    has_child = np.zeros(T, dtype=bool)
    has_child[parent[1:]] = True
    res = {
        "accept_len": np.zeros(B, np.int64), "best": np.zeros(B, np.int64),
        "next_tok": np.zeros(B, np.int64),
        "accepted_tok": np.full((B, Dm + 1), -1, np.int64),
        "p": np.full((B, T), np.nan), "thr": np.full((B, T), np.nan),
        "dec": np.zeros((B, T), bool), "acc": np.zeros((B, T), bool),
    }
    for b in range(B):
        P = {}
        thr = {}
        for n in range(T):
            if has_child[n]:
                Pn, Hn, _ = row_distribution(logits[b, n], temperature)
                P[n] = Pn
                thr[n] = min(eps, delta * math.exp(-Hn))
        acc = np.zeros(T, dtype=bool)
        acc[0] = True
        for c in range(1, T):
            n = parent[c]
            p = P[n][tree_tok[b, c]]
            dec = p > thr[n]
            res["p"][b, c] = p
            res["thr"][b, c] = thr[n]
            res["dec"][b, c] = dec
            acc[c] = acc[n] and dec
        alen = int(depth[acc].max())
        best = int(np.flatnonzero(acc & (depth == alen))[0])
        chain = []
        j = best
        while j != -1:
            chain.append(j)
            j = parent[j]
        chain.reverse()
        res["acc"][b] = acc
        res["accept_len"][b] = alen
        res["best"][b] = best
        res["accepted_tok"][b, :len(chain)] = tree_tok[b, chain]
        res["next_tok"][b] = int(np.argmax(logits[b, best]))
    return res


# ----------------------------------------------------------------------------
# (4b) rejection-sampling acceptance -- [P3] "两个扩展" and "关键发现":
#      typical acceptance is presented as the replacement for rejection
#      sampling (the comparison point); the pages do not spell the rule out.
# ----------------------------------------------------------------------------
def rs_accept_prob(p, q, x):
    """Probability of keeping a drafted token x: min(1, p(x) / q(x)), with
    p the target (verification) distribution and q the draft (head)
    distribution; q(x) = 0 keeps x iff p(x) > 0."""
    px, qx = float(p[x]), float(q[x])
    if qx == 0.0:
        return 1.0 if px > 0.0 else 0.0
    return min(1.0, px / qx)


def rs_residual(p, q):
    """Target after a rejected draft: max(0, p - q), renormalised.  When p <= q
    everywhere (then every draft is kept with probability 1, so a rejection
    cannot have happened) p is returned unchanged."""
    r = np.maximum(p - q, 0.0)
    Z = r.sum()
    return r / Z if Z > 0.0 else p


def sample_inverse_cdf(p, u):
    """Smallest token v with sum_{w <= v} p(w) > u * sum(p) (u in [0, 1)); the
    last token of nonzero probability if rounding leaves none."""
    c = np.cumsum(p)
    hit = np.flatnonzero(c > u * c[-1])
    return int(hit[0]) if hit.size else int(np.flatnonzero(p > 0)[-1])


def rejection_accept(logits, head_logits, tree_tok, tree, temperature, u_node, u_bonus):
    """Rejection-sampling acceptance over the candidate tree, per sequence.

    Reading (the standard speculative-sampling rule, extended to several
    drafts per node by testing siblings one after the other against the
    residual of the rejected ones): starting at the root (always kept), the
    children of the current node u are tried in rank order; child c with
    token x is kept iff u_node[b][c] < min(1, p(x) / q(x)), where p is the
    verification distribution at u (after the residual updates of the
    siblings rejected before c) and q is the distribution of the head that
    drafted c's depth (head depth(u), softmax of head_logits[depth(u)][b]),
    both at the given temperature.  A rejected sibling replaces p by
    rs_residual(p, q).  The first kept child becomes u; when none is kept, or
    u is a leaf, the step ends and the next token is sampled by inverse CDF
    with u_bonus[b] from the current p (the residual after all of u's
    children were rejected, else u's own distribution).  temperature 0 uses
    one-hot distributions at the argmax (lowest index), which makes this
    greedy verification.

    logits [B][T][V]; head_logits [K][B][V]; tree_tok [B][T];
    u_node [B][T], u_bonus [B] in [0, 1).
    Returns accept_len, best, next_tok, accepted_tok (as typical_accept) and
    a [B][T]: the keep probability of every tested node (nan elsewhere).
    """
    logits = np.asarray(logits, dtype=np.float64)
    head_logits = np.asarray(head_logits, dtype=np.float64)
    B, T, V = logits.shape
    parent, depth = tree["parent"], tree["depth"]
    Dm = tree["depth_max"]
    children = [[] for _ in range(T)]
    for c in range(1, T):
        children[parent[c]].append(c)            # increasing index = rank order
    res = {
        "accept_len": np.zeros(B, np.int64), "best": np.zeros(B, np.int64),
        "next_tok": np.zeros(B, np.int64),
        "accepted_tok": np.full((B, Dm + 1), -1, np.int64),
        "a": np.full((B, T), np.nan),
    }
    for b in range(B):
        u, chain = 0, [0]
        while True:
            p, _, _ = row_distribution(logits[b, u], temperature)
            if not children[u]:
                break
            q, _, _ = row_distribution(head_logits[depth[u], b], temperature)
            kept = None
            for c in children[u]:
                a = rs_accept_prob(p, q, int(tree_tok[b, c]))
                res["a"][b, c] = a
                if u_node[b, c] < a:
                    kept = c
                    break
                p = rs_residual(p, q)
            if kept is None:
                break
            u = kept
            chain.append(u)
        res["accept_len"][b] = depth[u]
        res["best"][b] = u
        res["accepted_tok"][b, :len(chain)] = np.asarray(tree_tok)[b, chain]
        res["next_tok"][b] = sample_inverse_cdf(p, float(u_bonus[b]))
    return res


# ----------------------------------------------------------------------------
# (5) KV-cache commit -- [P3] "基准/方法设计" (the next round starts after the
#     accepted prefix), [P2] "部署与生成" (generation keeps the KV cache)
# ----------------------------------------------------------------------------
def kv_commit(tree, k_tree, v_tree, best, seq_len, k_cache, v_cache):
    """Append each sequence's accepted path to its prefix cache.

    The accepted tokens are the path root..best; keeping their keys and values
    lets the next step treat them as ordinary prefix tokens.  Reading: node j
    of the path is written at its tree position seq_len[b] + depth(j)
    (tree_positions), so the cache holds prefix, root, ..., best in order;
    rows that would pass the cache capacity L_cap are dropped; a sequence
    whose best is not a node, or whose length is outside [0, L_cap], is left
    unchanged.
    k_tree, v_tree [B][T][nh][dh]; k_cache, v_cache [B][nh][L_cap][dh];
    best, seq_len [B].  Returns new (k_cache, v_cache, seq_len) (copies).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    lens = np.array(seq_len, dtype=np.int64, copy=True)
    B, T = k_tree.shape[0], k_tree.shape[1]
    L_cap = kc.shape[2]
    for b in range(B):
        j, L = int(best[b]), int(lens[b])
        if not (0 <= j < T and 0 <= L <= L_cap):
            continue
        pos = tree_positions(tree, L)
        path = ancestors(tree, j)             # root .. j, increasing depth
        n = 0
        for node in path:
            p = int(pos[node])
            if p >= L_cap:
                break
            kc[b, :, p] = k_tree[b, node]
            vc[b, :, p] = v_tree[b, node]
            n += 1
        lens[b] = L + n
    return kc, vc, lens


# ----------------------------------------------------------------------------
# the whole step
# ----------------------------------------------------------------------------
def topk_per_head(logits, k):
    """medusa_topk applied to each head's [M][V] block: returns idx [K][M][k], val [K][M][k]."""
    K, M, V = logits.shape
    idx, val = medusa_topk(logits.reshape(K * M, V), k)
    return idx.reshape(K, M, k), val.reshape(K, M, k)


def step(h, W1, W2, root_tok, tree, k, q, k_tree, v_tree, k_cache, v_cache,
         verify_logits, eps, delta, temperature=1.0, round_r_bf16=False,
         scale=None, attn_sel=None):
    """One verify tree-step in the order the pages give: heads -> top-k ->
    candidate tokens -> tree attention -> typical acceptance.
    verify_logits(tree_tok) supplies the backbone's logits at every tree
    node (the backbone itself is outside this path); it may also be an
    array [B][T][V]."""
    logits = medusa_heads(h, W1, W2, round_r_bf16)
    idx, val = topk_per_head(logits, k)
    tok = tree_tokens(tree, root_tok, idx)
    attn = tree_attention(q, k_tree, v_tree, k_cache, v_cache, tree, scale, attn_sel)
    vl = verify_logits(tok) if callable(verify_logits) else verify_logits
    acc = typical_accept(vl, tok, tree, eps, delta, temperature)
    return {"head_logits": logits, "topk_idx": idx, "topk_val": val,
            "tree_tok": tok, "attn": attn, "accept": acc}

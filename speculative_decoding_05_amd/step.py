"""One Medusa verify tree-step on the GPU, assembled from the C-ABI calls.

heads -> per-head top-k -> tree tokens -> tree attention -> typical
acceptance, all enqueued on torch's current stream with preallocated
buffers and workspaces (nothing is allocated inside `run`).
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as mb
from . import configs, synth


def to_device(a, device="cuda") -> torch.Tensor:
    """Upload a synth tensor (uint16 bf16 bit patterns or float32 / int32), or
    copy a torch tensor to `device` (always a new tensor)."""
    if isinstance(a, torch.Tensor):
        return a.to(device, copy=True)
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def build_tree(cfg: configs.Config) -> mb.Tree:
    """The configuration's candidate tree, built by the library."""
    spec = cfg.tree
    if spec.kind == "dense":
        paths = mb.dense_paths(cfg.K, spec.k)
    else:
        acc = np.array([[configs.acc_float(d, i) for i in range(spec.rank_cap)] for d in range(cfg.K)])
        paths = mb.greedy_paths(acc, spec.n_paths)
    return mb.Tree(paths, cfg.K, spec.k).upload()


def uses_tile_max(cfg: configs.Config) -> bool:
    """Whether a step takes the top-k from the vocabulary projection's tile maxima.

    The projection then writes one 4-byte image per 16 logits of each row,
    scattered over the rows, and the top-k reads those images and a dozen
    tiles per row instead of the whole row (about 6.9 -> 4.7 us per call).
    Measured per step on MI355X: 1.7 us faster at one row; at 8 and 32 rows
    the scattered image writes cost the projection 3.6-5.4 us, more than the
    top-k saves, and at 16 rows the two are within noise.  Two rows cause as
    many separate image writes per call as 16 rows do (there one block's
    eight adjacent images of a row go out together), so they are taken as
    break-even or better; two rows were not measured.
    """
    return cfg.dtype == "bf16" and cfg.B <= 2


class Step:
    """Device buffers of one configuration and the launch sequence of one step.

    `copies` > 1 keeps several copies of every per-step input (hidden state,
    tree Q/K/V, KV cache, verification logits) so that consecutive steps can
    rotate through them and not be served from the last-level cache.
    """

    def __init__(self, cfg: configs.Config, tree: mb.Tree, host: dict, copies: int = 1, device="cuda",
                 weights_of: "Step | None" = None):
        self.cfg, self.tree, self.copies = cfg, tree, copies
        B, K, V, H, k, T = cfg.B, cfg.K, cfg.V, cfg.H, cfg.k, tree.T
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        self.dt = dt
        dev = device
        self.packed = cfg.dtype == "bf16"
        if weights_of is not None:  # share another step's (identically shaped) head weights
            for name in ("W1p", "W2p") if self.packed else ("W1", "W2"):
                setattr(self, name, getattr(weights_of, name))
        else:
            self.W1 = to_device(host["W1"], dev)
            self.W2 = to_device(host["W2"], dev)
            if self.packed:  # one-time reorder into the matrix-core fragment order
                group = mb.medusa_pack_group_for_rows(B)   # the heads see B rows per step
                self.W1p = mb.PackedWeights(self.W1, group)
                self.W2p = mb.PackedWeights(self.W2, group)
                torch.cuda.synchronize()
                del self.W1, self.W2
        rt = host["root_tok"]
        self.root = to_device(rt.to(torch.int32) if isinstance(rt, torch.Tensor) else rt.astype(np.int32), dev)
        self.h = [to_device(host["h"], dev) for _ in range(copies)]
        self.q = [to_device(host["q"], dev) for _ in range(copies)]
        self.kt = [to_device(host["kt"], dev) for _ in range(copies)]
        self.vt = [to_device(host["vt"], dev) for _ in range(copies)]
        self.kc = [to_device(host["kc"], dev) for _ in range(copies)]
        self.vc = [to_device(host["vc"], dev) for _ in range(copies)]
        self.vlogits = [None] * copies
        if host.get("vlogits") is not None:
            self.set_verify_logits(host["vlogits"])
        self.r = torch.empty((K, B, H), dtype=dt, device=dev)
        self.head_logits = torch.empty((K, B, V), dtype=torch.float32, device=dev)
        self.tile_max = (torch.empty((K, B, (V + 15) // 16), dtype=torch.int32, device=dev)
                         if uses_tile_max(cfg) else None)
        self.topk_idx = torch.empty((K, B, k), dtype=torch.int32, device=dev)
        self.tree_tok = torch.empty((B, T), dtype=torch.int32, device=dev)
        self.attn = torch.empty((B, T, cfg.nh, cfg.dh), dtype=dt, device=dev)
        self.accept_len = torch.empty(B, dtype=torch.int32, device=dev)
        self.best = torch.empty(B, dtype=torch.int32, device=dev)
        self.next_tok = torch.empty(B, dtype=torch.int32, device=dev)
        self.accepted = torch.empty((B, tree.depth_max + 1), dtype=torch.int32, device=dev)
        dcode = mb.BF16 if cfg.dtype == "bf16" else mb.F32
        self.ws_topk = mb.workspace(mb.medusa_topk_workspace(K * B, V, k), dev)
        self.ws_attn = mb.workspace(mb.tree_attention_workspace(dcode, tree, B, cfg.nh, cfg.dh, cfg.L), dev)
        self.ws_acc = mb.workspace(mb.typical_accept_workspace(tree, B, V), dev)

    def set_verify_logits(self, vl: np.ndarray):
        for i in range(self.copies):
            self.vlogits[i] = to_device(vl.astype(np.float32))

    # -- the stages -------------------------------------------------------------
    def heads(self, i=0):
        if self.packed:
            mb.medusa_head_resblock_packed(self.h[i], self.W1p, self.r)
        else:
            mb.medusa_head_resblock(self.h[i], self.W1, self.r)

    def heads_vocab(self, i=0):
        if self.tile_max is not None:
            mb.medusa_head_vocab_packed_tmax(self.r, self.W2p, self.head_logits, self.tile_max)
        elif self.packed:
            mb.medusa_head_vocab_packed(self.r, self.W2p, self.head_logits)
        else:
            mb.medusa_head_vocab(self.r, self.W2, self.head_logits)

    def topk_and_tokens(self, i=0):
        if self.tile_max is not None:
            mb.medusa_topk_tree_tokens_tmax(self.tree, self.head_logits, self.tile_max, self.cfg.k, self.root,
                                            self.topk_idx, self.tree_tok)
            return
        mb.medusa_topk_tree_tokens(self.tree, self.head_logits, self.cfg.k, self.root, self.topk_idx,
                                   self.tree_tok, self.ws_topk)

    def attention(self, i=0):
        mb.tree_attention(self.tree, self.q[i], self.kt[i], self.vt[i], self.kc[i], self.vc[i], self.attn,
                          0.0, self.ws_attn)

    def accept(self, i=0):
        c = self.cfg
        mb.typical_accept(self.tree, self.vlogits[i], self.tree_tok, c.eps, c.delta, c.temperature,
                          self.accept_len, self.best, self.next_tok, self.accepted, None, None, self.ws_acc)

    def run(self, i=0):
        """Enqueue one whole verify tree-step on the current stream."""
        self.heads(i)
        self.heads_vocab(i)
        self.topk_and_tokens(i)
        self.attention(i)
        self.accept(i)


class VerifyPass:
    """The verify pass's dense contractions over all M = B*T tree nodes (bf16):
    the Medusa heads on every node's hidden state, and the backbone's LM head
    (a head with W1 = 0) turning the tree-attention output of `step` into
    verification logits.  Inputs are seeded device-side normals."""

    def __init__(self, step: Step, seed: int = 0, h_nodes: np.ndarray | None = None,
                 W_lm: np.ndarray | None = None):
        cfg, T = step.cfg, step.tree.T
        if not step.packed:
            raise ValueError("the verify pass runs on the bf16 (packed-weight) path")
        self.step, self.M = step, cfg.B * T
        M, H, V, K = self.M, cfg.H, cfg.V, cfg.K
        g = torch.Generator(device="cuda").manual_seed(seed)
        # host arrays (synth bf16 bits) when given, else device-side normals
        if h_nodes is not None:
            self.h = to_device(h_nodes)
        else:
            self.h = torch.randn((M, H), generator=g, device="cuda").to(torch.bfloat16)
        if W_lm is not None:
            W_lm = to_device(W_lm).reshape(1, V, H)
        else:
            W_lm = (torch.randn((1, V, H), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        self.W_lm = mb.PackedWeights(W_lm, mb.medusa_pack_group_for_rows(M))
        torch.cuda.synchronize()
        del W_lm
        self.r = torch.empty((K, M, H), dtype=torch.bfloat16, device="cuda")
        self.logits = torch.empty((K, M, V), dtype=torch.float32, device="cuda")
        self.vlogits = torch.empty((1, M, V), dtype=torch.float32, device="cuda")
        # activations in fragment order for the many-row contractions (shared by the calls)
        self.ws = mb.workspace(max(mb.medusa_head_workspace(K, M, H), mb.medusa_heads_workspace(K, M, H)))

    def heads_resblock(self):
        mb.medusa_head_resblock_packed_ws(self.h, self.step.W1p, self.r, self.ws)

    def heads_vocab(self):
        mb.medusa_head_vocab_packed_ws(self.r, self.step.W2p, self.logits, self.ws)

    def heads(self):
        """ResBlock and vocabulary projection in one call (r not copied twice)."""
        mb.medusa_heads_packed_ws(self.h, self.step.W1p, self.step.W2p, self.r, self.logits, self.ws)

    def lm_head(self):
        c = self.step.cfg
        mb.medusa_head_vocab_packed_ws(self.step.attn.reshape(1, self.M, c.H), self.W_lm, self.vlogits, self.ws)


def host_inputs(cfg: configs.Config, T: int, B: int | None = None, L: int | None = None) -> dict:
    """All seeded inputs of a configuration except the verification logits."""
    W1, W2 = synth.head_weights(cfg)
    kc, vc = synth.kv_cache(cfg, B, L)
    q, kt, vt = synth.tree_qkv(cfg, T, B)
    return {"W1": W1, "W2": W2, "h": synth.hidden(cfg, B), "root_tok": synth.root_tokens(cfg, B),
            "q": q, "kt": kt, "vt": vt, "kc": kc, "vc": vc}


def device_inputs(cfg: configs.Config, T: int, seed: int = 0, device="cuda") -> dict:
    """Inputs of the same shapes and distributions as host_inputs (weights
    N(0, 0.02^2), activations and caches N(0, 1), rounded to the storage type;
    uniform root tokens), drawn on the device from torch's generator: for
    timing-only runs of the large workloads, where drawing on the host takes
    tens of seconds."""
    g = torch.Generator(device=device).manual_seed(seed)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    B, K, H, V, nh, dh, L = cfg.B, cfg.K, cfg.H, cfg.V, cfg.nh, cfg.dh, cfg.L

    def normal(shape, std=1.0):
        return (torch.randn(shape, generator=g, device=device) * std).to(dt)

    return {"W1": normal((K, H, H), 0.02), "W2": normal((K, V, H), 0.02), "h": normal((B, H)),
            "root_tok": torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int32),
            "q": normal((B, T, nh, dh)), "kt": normal((B, T, nh, dh)), "vt": normal((B, T, nh, dh)),
            "kc": normal((B, nh, L, dh)), "vc": normal((B, nh, L, dh))}


def verify_logits_for(cfg: configs.Config, tree: mb.Tree, topk_idx: np.ndarray, root_tok: np.ndarray):
    """Planted verification logits for the given top-k candidates (synthetic)."""
    return synth.verification_logits(cfg.cfg_id, cfg.V, tree.parent, tree.depth, tree.rank, topk_idx,
                                     root_tok, configs.acc_float, cfg.k)

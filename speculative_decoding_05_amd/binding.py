"""Thin Python binding over libmedusa_hip.so (the C ABI in include/medusa.h).

Argument marshalling only: every step of the verify tree-step runs in the
library's HIP kernels.  Device tensors are torch tensors on the current HIP
device; they are passed by data_ptr() together with torch's current stream.
Importing this module fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmedusa_hip.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m speculative_decoding_05_amd.build`")
lib = ctypes.CDLL(LIB_PATH)

OK, ERR_ARG, ERR_SHAPE, ERR_TREE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_STATE, ERR_NONFINITE = range(9)
STATUS_NAMES = ["OK", "ERR_ARG", "ERR_SHAPE", "ERR_TREE", "ERR_UNSUPPORTED", "ERR_WORKSPACE", "ERR_HIP", "ERR_STATE",
                "ERR_NONFINITE"]
F32, BF16 = 0, 1
MAX_TOPK, MAX_TREE = 64, 1024

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t
_ip = ctypes.POINTER(ctypes.c_int32)
_u64p = ctypes.POINTER(ctypes.c_uint64)

# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "medusa_last_error": (ctypes.c_char_p, []),
    "medusa_abi_version": (_i, []),
    "medusa_head_resblock": (_i, [_p, _i, _i, _i, _i, _p, _p, _p]),
    "medusa_head_vocab": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p]),
    "medusa_heads": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]),
    "medusa_packed_weight_bytes": (_sz, [_i, _i, _i]),
    "medusa_pack_group_for_rows": (_i, [_i]),
    "medusa_pack_weights": (_i, [_p, _i, _i, _i, _i, _p, _p]),
    "medusa_head_resblock_packed": (_i, [_p, _i, _i, _i, _i, _p, _p, _p]),
    "medusa_head_vocab_packed": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p]),
    "medusa_head_vocab_packed_tmax": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p]),
    "medusa_heads_packed": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p]),
    "medusa_head_workspace": (_sz, [_i, _i, _i]),
    "medusa_head_resblock_packed_ws": (_i, [_p, _i, _i, _i, _i, _p, _p, _p, _p, _sz]),
    "medusa_head_vocab_packed_ws": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _sz]),
    "medusa_heads_workspace": (_sz, [_i, _i, _i]),
    "medusa_heads_packed_ws": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz]),
    "medusa_topk_workspace": (_sz, [_i, _i, _i]),
    "medusa_topk": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _sz]),
    "medusa_dense_paths": (_i, [_i, _i, _i, _ip, _ip, ctypes.POINTER(_i)]),
    "medusa_greedy_paths": (_i, [ctypes.POINTER(ctypes.c_double), _i, _i, _i, _ip, _ip]),
    "medusa_build_tree": (_i, [_ip, _ip, _i, _i, _i, ctypes.POINTER(_p)]),
    "medusa_tree_mask": (_i, [_p, ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i),
                              ctypes.POINTER(_i), _u64p, _ip, _ip, _ip, _ip]),
    "medusa_tree_positions": (_i, [_p, _i, _ip]),
    "medusa_tree_upload": (_i, [_p]),
    "medusa_tree_free": (None, [_p]),
    "medusa_tree_tokens": (_i, [_p, _p, _i, _i, _i, _p, _p, _p]),
    "medusa_topk_tree_tokens": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _sz]),
    "medusa_topk_tree_tokens_tmax": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p]),
    "tree_attention_workspace": (_sz, [_i, _p, _i, _i, _i, _i]),
    "tree_attention": (_i, [_p, _i, _p, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "tree_attention_ragged": (_i, [_p, _i, _p, _i, _i, _i, _i, _i, _p, _f, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "medusa_kv_commit": (_i, [_p, _i, _p, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "rejection_accept": (_i, [_p, _p, _i, _i, _i, _p, _p, _p, _f, _p, _p, _p, _p, _p, _p, _p]),
    "typical_accept_workspace": (_sz, [_p, _i, _i]),
    "typical_accept": (_i, [_p, _p, _i, _i, _p, _p, _f, _f, _f, _p, _p, _p, _p, _p, _p, _p, _sz]),
    "typical_accept_noalloc": (_i, [_p, _p, _i, _i, _p, _p, _f, _f, _f, _p, _p, _p, _p, _p, _p]),
    "medusa_peak_hbm_read": (_i, [_p, _p, _sz, _p]),
    "medusa_peak_mfma_bf16": (_i, [_p, _i, _i, _p]),
    "medusa_peak_mfma_flops": (ctypes.c_double, [_i, _i]),
    "medusa_device_info": (_i, [ctypes.POINTER(_i), ctypes.POINTER(_i), ctypes.POINTER(_i)]),
}
for _name, (_res, _args) in SIGNATURES.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class MedusaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES[status] if 0 <= status < len(STATUS_NAMES) else status}: {msg}")
        self.status = status


def check(status):
    if status != OK:
        raise MedusaError(status, lib.medusa_last_error().decode(errors="replace"))


def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensor is not on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensor is not contiguous")


def workspace(nbytes, device=None):
    """Zero-filled device scratch buffer of at least nbytes (16-byte aligned)."""
    torch = _torch()
    return torch.zeros(max(int(nbytes), 16), dtype=torch.uint8, device=device or "cuda")


# ---------------------------------------------------------------- heads
def medusa_head_resblock(h, W1, r):
    _dev(h, W1, r)
    K, H = W1.shape[0], W1.shape[2]
    M = h.shape[0]
    check(lib.medusa_head_resblock(_stream(), _dtype_code(h), K, M, H, _ptr(h), _ptr(W1), _ptr(r)))
    return r


def medusa_head_vocab(r, W2, logits):
    _dev(r, W2, logits)
    K, V, H = W2.shape
    M = r.shape[1]
    check(lib.medusa_head_vocab(_stream(), _dtype_code(r), K, M, H, V, _ptr(r), _ptr(W2), _ptr(logits)))
    return logits


def medusa_heads(h, W1, W2, r, logits):
    _dev(h, W1, W2, r, logits)
    K, V, H = W2.shape
    M = h.shape[0]
    check(lib.medusa_heads(_stream(), _dtype_code(h), K, M, H, V, _ptr(h), _ptr(W1), _ptr(W2),
                           _ptr(r), _ptr(logits)))
    return logits


def medusa_pack_group_for_rows(M):
    return lib.medusa_pack_group_for_rows(M)


class PackedWeights:
    """bf16 head weights [K][N][H] reordered once into the matrix-core fragment
    order, row tiles interleaved in groups of `group` (1, 2, 4 or 8)."""

    def __init__(self, W, group=1):
        torch = _torch()
        _dev(W)
        if W.dtype != torch.bfloat16:
            raise TypeError("packed weights are bf16")
        self.K, self.N, self.H = W.shape
        self.group = int(group)
        nbytes = lib.medusa_packed_weight_bytes(self.K, self.N, self.H)
        self.data = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=W.device)
        check(lib.medusa_pack_weights(_stream(), self.K, self.N, self.H, self.group, _ptr(W), _ptr(self.data)))


def medusa_head_resblock_packed(h, W1p, r):
    _dev(h, r)
    check(lib.medusa_head_resblock_packed(_stream(), W1p.K, h.shape[0], W1p.H, W1p.group, _ptr(h), _ptr(W1p.data),
                                          _ptr(r)))
    return r


def medusa_head_vocab_packed(r, W2p, logits):
    _dev(r, logits)
    check(lib.medusa_head_vocab_packed(_stream(), W2p.K, r.shape[1], W2p.H, W2p.N, W2p.group, _ptr(r),
                                       _ptr(W2p.data), _ptr(logits)))
    return logits


def medusa_head_vocab_packed_tmax(r, W2p, logits, tile_max):
    """As medusa_head_vocab_packed, also writing tile_max [K][M][ceil(V/16)] (int32 tensor of uint32 images)."""
    _dev(r, logits, tile_max)
    check(lib.medusa_head_vocab_packed_tmax(_stream(), W2p.K, r.shape[1], W2p.H, W2p.N, W2p.group, _ptr(r),
                                            _ptr(W2p.data), _ptr(logits), _ptr(tile_max)))
    return logits


def medusa_heads_packed(h, W1p, W2p, r, logits):
    _dev(h, r, logits)
    if W1p.group != W2p.group:
        raise ValueError("W1p and W2p must share one packing group")
    check(lib.medusa_heads_packed(_stream(), W2p.K, h.shape[0], W2p.H, W2p.N, W2p.group, _ptr(h), _ptr(W1p.data),
                                  _ptr(W2p.data), _ptr(r), _ptr(logits)))
    return logits


def medusa_head_workspace(K, M, H):
    return lib.medusa_head_workspace(K, M, H)


def medusa_head_resblock_packed_ws(h, W1p, r, ws=None):
    _dev(h, r)
    M = h.shape[0]
    if ws is None:
        ws = workspace(lib.medusa_head_workspace(W1p.K, M, W1p.H), h.device)
    _dev(ws)
    check(lib.medusa_head_resblock_packed_ws(_stream(), W1p.K, M, W1p.H, W1p.group, _ptr(h), _ptr(W1p.data),
                                             _ptr(r), _ptr(ws), ws.numel() * ws.element_size()))
    return r


def medusa_head_vocab_packed_ws(r, W2p, logits, ws=None):
    _dev(r, logits)
    M = r.shape[1]
    if ws is None:
        ws = workspace(lib.medusa_head_workspace(W2p.K, M, W2p.H), r.device)
    _dev(ws)
    check(lib.medusa_head_vocab_packed_ws(_stream(), W2p.K, M, W2p.H, W2p.N, W2p.group, _ptr(r), _ptr(W2p.data),
                                          _ptr(logits), _ptr(ws), ws.numel() * ws.element_size()))
    return logits


def medusa_heads_workspace(K, M, H):
    return lib.medusa_heads_workspace(K, M, H)


def medusa_heads_packed_ws(h, W1p, W2p, r, logits, ws=None):
    _dev(h, r, logits)
    if W1p.group != W2p.group:
        raise ValueError("W1p and W2p must share one packing group")
    M = h.shape[0]
    if ws is None:
        ws = workspace(lib.medusa_heads_workspace(W2p.K, M, W2p.H), h.device)
    _dev(ws)
    check(lib.medusa_heads_packed_ws(_stream(), W2p.K, M, W2p.H, W2p.N, W2p.group, _ptr(h), _ptr(W1p.data),
                                     _ptr(W2p.data), _ptr(r), _ptr(logits), _ptr(ws), ws.numel() * ws.element_size()))
    return logits


# ---------------------------------------------------------------- top-k
def medusa_topk_workspace(R, V, k):
    return lib.medusa_topk_workspace(R, V, k)


def medusa_topk(logits, k, idx, val=None, ws=None):
    """logits [..., V] float32 -> idx [..., k] int32 (and val)."""
    _dev(logits, idx, val)
    V = logits.shape[-1]
    R = logits.numel() // V
    if ws is None:
        ws = workspace(medusa_topk_workspace(R, V, k), logits.device)
    check(lib.medusa_topk(_stream(), R, V, k, _ptr(logits), _ptr(idx), _ptr(val), _ptr(ws), ws.numel()))
    return idx


# ---------------------------------------------------------------- trees
def dense_paths(K, k):
    n = _i(0)
    check(lib.medusa_dense_paths(K, k, 0, None, None, ctypes.byref(n)))
    ranks = np.zeros(n.value * K, dtype=np.int32)
    lens = np.zeros(n.value, dtype=np.int32)
    check(lib.medusa_dense_paths(K, k, n.value, ranks.ctypes.data_as(_ip), lens.ctypes.data_as(_ip),
                                 ctypes.byref(n)))
    return [tuple(ranks[p * K:p * K + lens[p]].tolist()) for p in range(n.value)]


def greedy_paths(acc, n_paths):
    """acc: [K][rank_cap] per-head top-i accuracies (float64)."""
    acc = np.ascontiguousarray(acc, dtype=np.float64)
    K, cap = acc.shape
    ranks = np.zeros(max(1, n_paths) * K, dtype=np.int32)
    lens = np.zeros(max(1, n_paths), dtype=np.int32)
    check(lib.medusa_greedy_paths(acc.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), K, cap, n_paths,
                                  ranks.ctypes.data_as(_ip), lens.ctypes.data_as(_ip)))
    return [tuple(ranks[p * K:p * K + lens[p]].tolist()) for p in range(n_paths)]


class Tree:
    """A candidate tree built by medusa_build_tree (host arrays + device copy)."""

    def __init__(self, paths, K, k):
        n = len(paths)
        ranks = np.zeros(max(1, n) * K, dtype=np.int32)
        lens = np.zeros(max(1, n), dtype=np.int32)
        for i, p in enumerate(paths):
            p = list(p)
            lens[i] = len(p)
            ranks[i * K:i * K + min(len(p), K)] = p[:K]
        h = _p()
        check(lib.medusa_build_tree(ranks.ctypes.data_as(_ip), lens.ctypes.data_as(_ip), n, K, k,
                                    ctypes.byref(h)))
        self.handle = h
        self.K, self.k = K, k
        T, W, D, nl = _i(), _i(), _i(), _i()
        check(lib.medusa_tree_mask(h, ctypes.byref(T), ctypes.byref(W), ctypes.byref(D), ctypes.byref(nl),
                                   None, None, None, None, None))
        self.T, self.W, self.depth_max, self.n_leaves = T.value, W.value, D.value, nl.value
        self.mask = np.zeros((self.T, self.W), dtype=np.uint64)
        self.parent = np.zeros(self.T, dtype=np.int32)
        self.depth = np.zeros(self.T, dtype=np.int32)
        self.rank = np.zeros(self.T, dtype=np.int32)
        self.retrieve = np.zeros((self.n_leaves, self.depth_max + 1), dtype=np.int32)
        check(lib.medusa_tree_mask(h, None, None, None, None, self.mask.ctypes.data_as(_u64p),
                                   self.parent.ctypes.data_as(_ip), self.depth.ctypes.data_as(_ip),
                                   self.rank.ctypes.data_as(_ip), self.retrieve.ctypes.data_as(_ip)))
        self.uploaded = False

    def positions(self, L):
        pos = np.zeros(self.T, dtype=np.int32)
        check(lib.medusa_tree_positions(self.handle, L, pos.ctypes.data_as(_ip)))
        return pos

    def upload(self):
        if not self.uploaded:
            check(lib.medusa_tree_upload(self.handle))
            self.uploaded = True
        return self

    def free(self):
        if self.handle:
            lib.medusa_tree_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def medusa_tree_tokens(tree, root_tok, topk_idx, tree_tok):
    """root_tok [B], topk_idx [K][B][k] int32 -> tree_tok [B][T] int32."""
    _dev(root_tok, topk_idx, tree_tok)
    K, B, k = topk_idx.shape
    check(lib.medusa_tree_tokens(_stream(), tree.handle, B, K, k, _ptr(root_tok), _ptr(topk_idx),
                                 _ptr(tree_tok)))
    return tree_tok


def medusa_topk_tree_tokens(tree, logits, k, root_tok, topk_idx, tree_tok, ws=None):
    """logits [K][B][V] -> topk_idx [K][B][k] and tree_tok [B][T] in one pass."""
    _dev(logits, root_tok, topk_idx, tree_tok)
    K, B, V = logits.shape
    if ws is None:
        ws = workspace(medusa_topk_workspace(K * B, V, k), logits.device)
    check(lib.medusa_topk_tree_tokens(_stream(), tree.handle, B, K, V, k, _ptr(logits), _ptr(root_tok),
                                      _ptr(topk_idx), _ptr(tree_tok), _ptr(ws), ws.numel()))
    return tree_tok


def medusa_topk_tree_tokens_tmax(tree, logits, tile_max, k, root_tok, topk_idx, tree_tok):
    """medusa_topk_tree_tokens reading the tile maxima written with the logits."""
    _dev(logits, tile_max, root_tok, topk_idx, tree_tok)
    K, B, V = logits.shape
    check(lib.medusa_topk_tree_tokens_tmax(_stream(), tree.handle, B, K, V, k, _ptr(logits), _ptr(tile_max),
                                           _ptr(root_tok), _ptr(topk_idx), _ptr(tree_tok)))
    return tree_tok


# ---------------------------------------------------------------- attention
def tree_attention_workspace(dtype_code, tree, B, nh, dh, L):
    return lib.tree_attention_workspace(dtype_code, tree.handle, B, nh, dh, L)


def tree_attention(tree, q, k_tree, v_tree, k_cache, v_cache, out, scale=0.0, ws=None):
    """q/k_tree/v_tree [B][T][nh][dh], k_cache/v_cache [B][nh][L][dh] -> out [B][T][nh][dh]."""
    _dev(q, k_tree, v_tree, k_cache, v_cache, out, ws)
    B, T, nh, dh = q.shape
    L = k_cache.shape[2]
    dt = _dtype_code(q)
    if ws is None:
        ws = workspace(tree_attention_workspace(dt, tree, B, nh, dh, L), q.device)
    check(lib.tree_attention(_stream(), dt, tree.handle, B, nh, dh, L, float(scale), _ptr(q), _ptr(k_tree),
                             _ptr(v_tree), _ptr(k_cache) if L else None, _ptr(v_cache) if L else None,
                             _ptr(out), _ptr(ws), ws.numel()))
    return out


# ---------------------------------------------------------------- acceptance
def tree_attention_ragged(tree, q, k_tree, v_tree, k_cache, v_cache, seq_len, L_max, out, scale=0.0, ws=None):
    """As tree_attention with a cache of capacity L_cap = k_cache.shape[2] and
    per-sequence prefix lengths seq_len [B] (device int32, each <= L_max)."""
    _dev(q, k_tree, v_tree, k_cache, v_cache, seq_len, out, ws)
    B, T, nh, dh = q.shape
    L_cap = k_cache.shape[2]
    dt = _dtype_code(q)
    if ws is None:
        ws = workspace(tree_attention_workspace(dt, tree, B, nh, dh, L_max), q.device)
    check(lib.tree_attention_ragged(_stream(), dt, tree.handle, B, nh, dh, L_cap, L_max, _ptr(seq_len),
                                    float(scale), _ptr(q), _ptr(k_tree), _ptr(v_tree), _ptr(k_cache),
                                    _ptr(v_cache), _ptr(out), _ptr(ws), ws.numel()))
    return out


def kv_commit(tree, k_tree, v_tree, best_node, seq_len, k_cache, v_cache, next_tok=None, root_tok=None):
    """Append each sequence's accepted path (root..best_node) to its cache
    [B][nh][L_cap][dh] at seq_len; seq_len grows in place; root_tok <- next_tok."""
    _dev(k_tree, v_tree, best_node, seq_len, k_cache, v_cache, next_tok, root_tok)
    B, T, nh, dh = k_tree.shape
    check(lib.medusa_kv_commit(_stream(), _dtype_code(k_tree), tree.handle, B, nh, dh, k_cache.shape[2],
                               _ptr(k_tree), _ptr(v_tree), _ptr(best_node), _ptr(seq_len), _ptr(k_cache),
                               _ptr(v_cache), _ptr(next_tok), _ptr(root_tok)))


def typical_accept_workspace(tree, B, V):
    return lib.typical_accept_workspace(tree.handle, B, V)


def typical_accept(tree, logits, tree_tok, eps, delta, temperature, accept_len, best_node, next_tok,
                   accepted_tok, cand_p=None, row_thr=None, ws=None):
    _dev(logits, tree_tok, accept_len, best_node, next_tok, accepted_tok, cand_p, row_thr, ws)
    B, T, V = logits.shape
    if ws is None:
        ws = workspace(typical_accept_workspace(tree, B, V), logits.device)
    check(lib.typical_accept(_stream(), tree.handle, B, V, _ptr(logits), _ptr(tree_tok), float(eps),
                             float(delta), float(temperature), _ptr(accept_len), _ptr(best_node),
                             _ptr(next_tok), _ptr(accepted_tok), _ptr(cand_p), _ptr(row_thr), _ptr(ws),
                             ws.numel()))


def typical_accept_noalloc(tree, logits, tree_tok, eps, delta, temperature, accept_len, best_node, next_tok,
                           accepted_tok, cand_p=None, row_thr=None):
    """typical_accept with the library's own scratch (no workspace argument)."""
    _dev(logits, tree_tok, accept_len, best_node, next_tok, accepted_tok, cand_p, row_thr)
    B, T, V = logits.shape
    check(lib.typical_accept_noalloc(_stream(), tree.handle, B, V, _ptr(logits), _ptr(tree_tok), float(eps),
                                     float(delta), float(temperature), _ptr(accept_len), _ptr(best_node),
                                     _ptr(next_tok), _ptr(accepted_tok), _ptr(cand_p), _ptr(row_thr)))


def rejection_accept(tree, logits, head_logits, tree_tok, temperature, u_node, u_bonus, accept_len, best_node,
                     next_tok, accepted_tok, keep_prob=None):
    """Rejection-sampling acceptance: logits [B][T][V], head_logits [K][B][V],
    uniforms u_node [B][T] and u_bonus [B]."""
    _dev(logits, head_logits, tree_tok, u_node, u_bonus, accept_len, best_node, next_tok, accepted_tok, keep_prob)
    B, T, V = logits.shape
    check(lib.rejection_accept(_stream(), tree.handle, B, V, head_logits.shape[0], _ptr(logits), _ptr(head_logits),
                               _ptr(tree_tok), float(temperature), _ptr(u_node), _ptr(u_bonus), _ptr(accept_len),
                               _ptr(best_node), _ptr(next_tok), _ptr(accepted_tok), _ptr(keep_prob)))


# ---------------------------------------------------------------- measurement
def peak_hbm_read(buf, sink):
    """Read all of `buf` (device tensor, its storage bytes) once."""
    _dev(buf, sink)
    check(lib.medusa_peak_hbm_read(_stream(), _ptr(buf), buf.numel() * buf.element_size(), _ptr(sink)))


def peak_mfma_bf16(blocks, iters, sink):
    """One call of the bf16 matrix-core loop; returns its flop count."""
    _dev(sink)
    check(lib.medusa_peak_mfma_bf16(_stream(), int(blocks), int(iters), _ptr(sink)))
    return lib.medusa_peak_mfma_flops(int(blocks), int(iters))


def device_info():
    """(compute units, peak clock kHz, peak memory clock kHz) of the current device."""
    cu, ck, mk = _i(0), _i(0), _i(0)
    check(lib.medusa_device_info(ctypes.byref(cu), ctypes.byref(ck), ctypes.byref(mk)))
    return cu.value, ck.value, mk.value

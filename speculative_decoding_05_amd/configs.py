"""The five workload shapes the verify tree-step is tested and measured on.

Parameters only: no arithmetic of the method lives here.  Shapes follow
the Vicuna-7B / Vicuna-13B layer shapes the Medusa pages evaluate on
(hidden 4096 / 5120, 32 / 40 heads of 128, vocabulary 32000), with
synthetic seeded data in place of checkpoints.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from fractions import Fraction

# Synthetic per-head top-i accuracy used to grow the sparse trees and to
# plant the verification logits: a(k, i) = 0.6 * 0.8**k * 0.5**i, k the
# 0-based head, i the 0-based rank.  Kept as exact rationals.
ACC_A0 = Fraction(3, 5)
ACC_RK = Fraction(4, 5)
ACC_RI = Fraction(1, 2)


def acc_exact(k: int, i: int) -> Fraction:
    return ACC_A0 * ACC_RK ** k * ACC_RI ** i


def acc_float(k: int, i: int) -> float:
    return float(acc_exact(k, i))


@dataclass(frozen=True)
class TreeSpec:
    kind: str            # "dense" or "greedy"
    k: int               # per-head top-k width
    n_paths: int = 0     # greedy: number of non-root nodes
    rank_cap: int = 0    # greedy: ranks considered per head


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int
    dtype: str           # "f32" or "bf16"
    B: int
    H: int
    nh: int
    dh: int
    V: int
    L: int
    K: int
    tree: TreeSpec
    eps: float = 0.09    # posterior_threshold
    delta: float = 0.3   # posterior_alpha
    temperature: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def k(self) -> int:
        return self.tree.k


GREEDY64 = TreeSpec("greedy", k=10, n_paths=63, rank_cap=10)

CONFIGS = {
    "tiny_f32": Config(
        "tiny_f32", 1, "f32", B=1, H=256, nh=4, dh=64, V=1000, L=128, K=2,
        tree=TreeSpec("dense", k=2),
        note="tiny fp32: dense top-2 tree of 7 nodes"),
    "vicuna7b_b1": Config(
        "vicuna7b_b1", 2, "bf16", B=1, H=4096, nh=32, dh=128, V=32000, L=1024,
        K=4, tree=GREEDY64,
        note="7B shape, batch 1, 64-node greedy sparse tree"),
    "roofline_b16": Config(
        "roofline_b16", 3, "bf16", B=16, H=4096, nh=32, dh=128, V=32000,
        L=1024, K=4, tree=GREEDY64,
        note="7B shape, batch 16, KV 1024, 64-node tree"),
    "vicuna13b_b8": Config(
        "vicuna13b_b8", 4, "bf16", B=8, H=5120, nh=40, dh=128, V=32000,
        L=4096, K=5, tree=GREEDY64,
        note="13B shape, batch 8, KV 4096, 64-node tree"),
    "dense341_b32": Config(
        "dense341_b32", 5, "bf16", B=32, H=4096, nh=32, dh=128, V=32000,
        L=2048, K=4, tree=TreeSpec("dense", k=4),
        note="7B shape, batch 32, KV 2048, dense top-4 tree of 341 nodes"),
}

ORDER = ["tiny_f32", "vicuna7b_b1", "roofline_b16", "vicuna13b_b8", "dense341_b32"]

"""The five workload shapes of the GDN tree-verify path.

Shapes follow the DFlash + DDTree decoder described on the GreenGames page
(hackdot.org/~GreenGames): a 27B GDN-hybrid target whose 48 linear-attention
layers use 48 value heads over 16 key heads of width 128 (section "Why the
experiment exists": 48 of 64 layers are Gated DeltaNet), a DDTree budget of 22
(TL;DR) and a drafting block of 16 tokens (section "Prefill"), which bounds
tree depth.  The verify step sees budget + 1 nodes: the root (the last
committed token) plus the drafts, which is the row count of the verify logits
buffer discussed in "Key wins".
"""
from __future__ import annotations

from dataclasses import dataclass

BASE_SEED = 20261203


@dataclass(frozen=True)
class Config:
    name: str
    index: int
    num_seqs: int
    num_layers: int
    num_k_heads: int
    num_v_heads: int
    head_dim: int
    dtype: str            # storage dtype of q/k/v: "f32" or "bf16"; gates/state are f32
    tree: tuple           # ("random", n, max_depth) | ("chain", n) | ("ddtree", budget, width, dmax)
    accept: str           # "leaf" | "chain_len" | "node"
    prefill_steps: int    # chain steps from a zero state that make the committed state
    num_slots: int
    slot_perm: bool       # slot_idx is a seeded permutation (else identity)
    max_depth: int = 16   # depth limit passed to the library (nodes on a root path)

    @property
    def seed(self) -> int:
        return BASE_SEED + self.index

    @property
    def max_nodes(self) -> int:
        kind = self.tree[0]
        if kind == "random":
            return self.tree[1]
        if kind == "chain":
            return self.tree[1]
        return self.tree[1] + 1  # budget drafts + root


CONFIGS = {
    # 1 sequence, 2 heads, d=16, fp32 inputs, 7-node random tree of depth <= 4.
    "tiny": Config("tiny", 0, 1, 1, 2, 2, 16, "f32", ("random", 7, 4), "leaf", 8, 1, False, 16),
    # W=1 linear verify over a 16-token block.
    "chain": Config("chain", 1, 1, 1, 16, 48, 128, "bf16", ("chain", 16), "chain_len", 64, 1, False, 16),
    # One DDTree of budget 22 (23 nodes), branching <= 4, depth <= 16.
    "ddtree22": Config("ddtree22", 2, 1, 1, 16, 48, 128, "bf16", ("ddtree", 22, 4, 16), "node", 64, 1, False, 16),
    # 32 sequences, each its own budget-22 tree, 32-slot cache addressed by a permutation.
    "batched": Config("batched", 3, 32, 1, 16, 48, 128, "bf16", ("ddtree", 22, 4, 16), "node", 64, 32, True, 16),
    # 64 sequences x 48 layers, budget-64 trees (branching <= 8), ~9.7 GB of state.
    "stress": Config("stress", 4, 64, 48, 16, 48, 128, "bf16", ("ddtree", 64, 8, 16), "node", 64, 64, True, 16),
}

ALIASES = {"c0": "tiny", "c1": "chain", "c2": "ddtree22", "c3": "batched", "c4": "stress"}


def get_config(name: str) -> Config:
    key = ALIASES.get(name.lower(), name.lower())
    return CONFIGS[key]

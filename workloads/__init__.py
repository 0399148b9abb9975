"""Seeded synthetic workloads for the GDN tree-verify / persist path.

This package only draws random numbers and arranges them into the shapes the
path consumes (draft trees, per-node q/k/v/gates, prefill tokens, accepted
nodes, cache slots). It contains none of the gated-delta-rule arithmetic, so
both the GPU library's tests/bench and the CPU oracle can use it without
sharing any of the method's code.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .trees import ddtree_tree, chain_tree, random_tree, relabel, tree_depths  # noqa: F401
from .inputs import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_accepts,
    make_layer_inputs,
    make_prefill,
    make_slots,
    make_trees,
    cu_from_trees,
)

"""Seeded synthetic workloads: determinism, shapes and tree limits (CPU only)."""
import numpy as np
import pytest
import torch

import workloads as W
from workloads.trees import tree_depths


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # ties go to even
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name", ["tiny", "chain", "ddtree22", "batched", "stress"])
def test_trees_respect_limits(name):
    cfg = W.get_config(name)
    trees = W.make_trees(cfg)
    assert len(trees) == cfg.num_seqs
    for par in trees:
        n = len(par)
        assert n == cfg.max_nodes
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, n))
        depth = tree_depths(par)
        assert depth.max() <= (cfg.tree[2] if cfg.tree[0] == "random" else cfg.max_depth)
        if cfg.tree[0] == "ddtree":
            width = cfg.tree[2]
            assert np.bincount(par[1:], minlength=n).max() <= width
            # chain pre-seed: nodes 1..15 extend the rank-1 chain
            assert list(par[1:16]) == list(range(0, 15))
    again = W.make_trees(cfg)
    assert all(np.array_equal(x, y) for x, y in zip(trees, again))


def test_inputs_deterministic_and_normalized():
    cfg = W.get_config("ddtree22")
    trees = W.make_trees(cfg)
    x = W.make_layer_inputs(cfg, 0, trees)
    y = W.make_layer_inputs(cfg, 0, trees)
    for key in x:
        assert np.array_equal(x[key], y[key])
    assert x["q"].dtype == np.uint16 and x["q"].shape == (23, 16, 128)
    assert x["v"].shape == (23, 48, 128) and x["a"].shape == (23, 48)
    k = W.bf16_bits_to_f32(x["k"]).astype(np.float64)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=1e-2)
    assert (x["a"] > 0).all() and (x["a"] < 1).all() and (x["b"] > 0).all() and (x["b"] < 1).all()
    other = W.make_layer_inputs(cfg, 1, trees)
    assert not np.array_equal(x["v"], other["v"])


def test_accepts_and_slots():
    cfg = W.get_config("batched")
    trees = W.make_trees(cfg)
    acc = W.make_accepts(cfg, trees)
    assert ((acc >= 0) & (acc < 23)).all()
    slots = W.make_slots(cfg)
    assert sorted(slots.tolist()) == list(range(32))
    c1 = W.get_config("chain")
    acc1 = W.make_accepts(c1, W.make_trees(c1))
    assert 0 <= acc1[0] < 16
    c0 = W.get_config("tiny")
    t0 = W.make_trees(c0)
    a0 = W.make_accepts(c0, t0)
    assert a0[0] not in set(t0[0][t0[0] >= 0].tolist())  # a leaf

"""The fp64 oracle against facts fixed by the mathematics (CPU only)."""
import numpy as np
import pytest

import oracle
import pins
from pins import golden_example


@pytest.mark.parametrize("pin", [
    pins.pin_tiny_unrolled, pins.pin_closed_forms, pins.pin_chain_equals_sequential,
    pins.pin_superposition, pins.pin_duplicate_siblings, pins.pin_ancestor_only,
    pins.pin_permutation, pins.pin_persist_replay, pins.pin_forest, pins.pin_batch_wrappers,
], ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_brute_force_all_small_trees():
    # 720 labeled trees of 7 nodes with parent[i] < i; those of depth <= 4
    checked = pins.pin_brute_force_small_trees(d=4)
    assert checked == 568  # counted independently: increasing trees on 7 nodes, height <= 3 edges


def test_exact_rational_example():
    """The hand-worked 2x2 example of tests/golden/rule_2x2_worked_example.json: every
    number is exact in binary, so fp64 must reproduce the hand-derived states and
    outputs exactly."""
    ex = golden_example()
    nodes = ex["nodes"]
    parent = np.array([nd["parent"] for nd in nodes], np.int32)
    vec = lambda key: np.array([[nd[key]] for nd in nodes])          # [node][head][dim]
    gate = lambda key: np.array([[nd[key]] for nd in nodes])         # [node][head]
    out, st = oracle.tree(parent, vec("q"), vec("k"), vec("v"), gate("a"), gate("b"),
                          np.array([ex["S0"]]), return_states=True)
    for i, nd in enumerate(nodes):
        assert np.array_equal(st[i, 0], nd["state"]), i
        assert np.array_equal(out[i, 0], nd["o"]), i


def test_initial_state_is_prefill_recurrence():
    """The committed state is the sequential recurrence over prefill tokens."""
    import workloads as W
    cfg = W.get_config("tiny")
    pre = W.make_prefill(cfg, 0)
    S0 = oracle.initial_states(pre, cfg.num_v_heads, cfg.head_dim)
    assert S0.dtype == np.float32 and S0.shape == (1, 2, 16, 16)
    from oracle.literal import literal_rule
    for h in range(2):
        S = np.zeros((16, 16))
        for t in range(cfg.prefill_steps):
            S = literal_rule(S, oracle.widen(pre["k"][0, t, h]), oracle.widen(pre["v"][0, t, h]),
                             float(pre["a"][0, t, h]), float(pre["b"][0, t, h]))
        assert np.array_equal(S.astype(np.float32), S0[0, h]) or pins.rel(S0[0, h], S) < 1e-7

"""The fp64 oracle against facts fixed by the mathematics (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", [
    pins.pin_tiny_unrolled, pins.pin_closed_forms, pins.pin_chain_equals_sequential,
    pins.pin_superposition, pins.pin_duplicate_siblings, pins.pin_ancestor_only,
    pins.pin_permutation, pins.pin_persist_replay, pins.pin_forest,
], ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_brute_force_all_small_trees():
    # 720 labeled trees of 7 nodes with parent[i] < i; those of depth <= 4
    checked = pins.pin_brute_force_small_trees(d=4)
    assert checked == 568  # counted independently: increasing trees on 7 nodes, height <= 3 edges


def test_exact_rational_example():
    """A 2x2 example whose every number is exact in binary, so fp64 must
    reproduce the hand-derived result exactly.

    S0 = [[1, 2], [3, 4]], k = (1, 0), v = (2, -2), a = 1/2, b = 1/4, q = (1, 1):
      S0 (I - b k k^T) = [[3/4, 2], [9/4, 4]]
      a * that         = [[3/8, 1], [9/8, 2]]
      + b v k^T        = [[3/8 + 1/2, 1], [9/8 - 1/2, 2]] = [[7/8, 1], [5/8, 2]]
      o = S' q         = (15/8, 21/8).
    A child with k = (0, 1), v = (1, 1), a = 1, b = 1/2, q = (0, 1):
      S' (I - b k k^T) = [[7/8, 1/2], [5/8, 1]];  + b v k^T = [[7/8, 1], [5/8, 3/2]]
      o = (1, 3/2)."""
    S0 = np.array([[[1.0, 2.0], [3.0, 4.0]]])
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    v = np.array([[[2.0, -2.0]], [[1.0, 1.0]]])
    q = np.array([[[1.0, 1.0]], [[0.0, 1.0]]])
    a = np.array([[0.5], [1.0]])
    b = np.array([[0.25], [0.5]])
    out, st = oracle.tree(np.array([-1, 0], np.int32), q, k, v, a, b, S0, return_states=True)
    assert np.array_equal(st[0, 0], [[7 / 8, 1.0], [5 / 8, 2.0]])
    assert np.array_equal(out[0, 0], [15 / 8, 21 / 8])
    assert np.array_equal(st[1, 0], [[7 / 8, 1.0], [5 / 8, 1.5]])
    assert np.array_equal(out[1, 0], [1.0, 1.5])


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

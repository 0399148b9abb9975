"""Pins of the draft top-k and DDTree builder oracle (``oracle/ddtree.py``)
against facts that do not depend on its code.

Each ``pin_*(impl)`` takes a module with the oracle's ``draft_topk``,
``build_tree`` and ``tree_size`` and raises AssertionError when it breaks the
fact it checks; ``tests/test_oracle_ddtree.py`` runs them on the real oracle
and on copies with a planted mistake.

The builder pin rests on a global characterization.  Scores only fall along a
path (log-probabilities are <= 0 and each level's candidates come in
descending order), so growing the tree best first, one candidate at a time,
takes nodes in one fixed total order.  The pin enumerates EVERY node the depth
and width limits allow, sorts them by that order -- higher score, then smaller
depth, then smaller rank, then the parent's own place in the order (the
pre-seeded chain first) -- and requires the built tree to be the rank-1 chain
followed by the first remaining nodes of that list, id for id.
"""
from __future__ import annotations

import itertools
import math

import numpy as np


def _levels(rng, L, W, ties: bool):
    """Descending log-probabilities [L][W] (ties: drawn from a small set)."""
    if ties:
        lp = -rng.choice([0.25, 0.5, 1.0, 1.5], size=(L, W))
    else:
        z = rng.normal(0.0, 2.0, size=(L, W))
        lp = z - np.log(np.exp(z).sum(axis=1, keepdims=True))
    lp = -np.sort(-lp, axis=1)
    return lp.astype(np.float32)


def brute_force_tree(root_token, tokens, lp, budget, max_depth=16):
    L, W = tokens.shape
    cap = min(L + 1, max_depth)
    lp = np.asarray(lp, dtype=np.float32)
    chain = [()]
    while len(chain) - 1 < budget and len(chain) < cap:
        chain.append(chain[-1] + (0,))
    chain_pos = {p: i for i, p in enumerate(chain)}
    score = {(): np.float32(0.0)}
    nodes = []
    for d in range(1, cap):
        for path in itertools.product(range(W), repeat=d):
            score[path] = np.float32(score[path[:-1]] + lp[d - 1, path[-1]])
            nodes.append(path)
    keys = {}

    def key(path):
        if path in chain_pos:
            return (0, chain_pos[path])
        if path not in keys:
            keys[path] = (1, -float(score[path]), len(path) + 1, path[-1], key(path[:-1]))
        return keys[path]

    rest = sorted((p for p in nodes if p not in chain_pos), key=key)
    order = chain + rest[: max(0, budget - (len(chain) - 1))]
    ids = {p: i for i, p in enumerate(order)}
    parent = np.array([-1] + [ids[p[:-1]] for p in order[1:]], dtype=np.int32)
    token = np.array([root_token] + [int(tokens[len(p) - 1, p[-1]]) for p in order[1:]], dtype=np.int32)
    return parent, token


def pin_builder_is_global_order(impl):
    rng = np.random.default_rng(21)
    cases = [(4, 2, 9), (3, 3, 20), (5, 2, 40), (3, 4, 60), (2, 5, 30), (6, 1, 4), (6, 2, 200), (4, 3, 5)]
    for trial, (L, W, budget) in enumerate(cases * 3):
        ties = trial % 2 == 0
        lp = _levels(rng, L, W, ties)
        tokens = rng.integers(0, 1000, size=(L, W))
        max_depth = 16 if trial % 3 else min(16, L)  # sometimes the depth limit binds before L
        par, tok, _ = impl.build_tree(7, tokens, lp, budget, max_depth)
        ep, et = brute_force_tree(7, tokens, lp, budget, max_depth)
        assert np.array_equal(par, ep) and np.array_equal(tok, et), (trial, L, W, budget, par, ep)
        assert len(par) == impl.tree_size(L, W, budget, max_depth)


def pin_builder_limits(impl):
    """Budget, width and depth limits; parents precede children; the chain."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        L = int(rng.integers(1, 15))
        W = int(rng.integers(1, 6))
        budget = int(rng.integers(0, 80))
        lp = _levels(rng, L, W, bool(rng.integers(2)))
        tokens = rng.integers(0, 50, size=(L, W))
        par, tok, _ = impl.build_tree(3, tokens, lp, budget)
        n = len(par)
        cap = sum(W ** d for d in range(1, L + 1))
        assert n == 1 + min(budget, cap)
        assert par[0] == -1 and all(0 <= par[i] < i for i in range(1, n))
        depth = [1] * n
        for i in range(1, n):
            depth[i] = depth[par[i]] + 1
        assert max(depth) <= L + 1
        kids = np.bincount(par[1:], minlength=n) if n > 1 else np.zeros(1, int)
        assert kids.max(initial=0) <= W
        s = min(budget, L)
        assert list(par[1:s + 1]) == list(range(s)) and all(tok[i] == tokens[i - 1, 0] for i in range(1, s + 1))


def pin_topk_is_stable_sort(impl):
    """Without NaNs the candidates are numpy's stable descending sort (equal
    values keep the smaller id; +0 and -0 are equal)."""
    rng = np.random.default_rng(2)
    for V in (1, 3, 17, 300):
        x = rng.choice(np.array([-1.0, -0.0, 0.0, 0.5, 2.0, -np.inf, np.inf], dtype=np.float32), size=(6, V))
        x[:3] = rng.standard_normal((3, V)).astype(np.float32)
        for W in (1, 4, 8):
            tok, _ = impl.draft_topk(x, W)
            for r in range(len(x)):
                w = min(W, V)
                want = np.argsort(-x[r].astype(np.float64), kind="stable")[:w]
                assert np.array_equal(tok[r, :w], want), (V, W, r, tok[r], want)
                assert (tok[r, w:] == -1).all()


def pin_topk_logp_closed_forms(impl):
    V = 64
    tok, lp = impl.draft_topk(np.zeros((1, V), dtype=np.float32), 4)
    assert np.allclose(lp[0], -math.log(V), atol=1e-12, rtol=0) and list(tok[0]) == [0, 1, 2, 3]
    x = np.full((1, V), -np.inf, dtype=np.float32)
    x[0, 9], x[0, 40] = 3.0, 1.0
    tok, lp = impl.draft_topk(x, 3)
    lse = 3.0 + math.log(1.0 + math.exp(-2.0))
    assert list(tok[0]) == [9, 40, 0]
    assert abs(lp[0, 0] - (3.0 - lse)) < 1e-12 and abs(lp[0, 1] - (1.0 - lse)) < 1e-12 and lp[0, 2] == -np.inf
    # a whole small vocabulary: the probabilities sum to one
    x = np.random.default_rng(0).standard_normal((3, 6)).astype(np.float32)
    _, lp = impl.draft_topk(x, 6)
    assert np.allclose(np.exp(lp).sum(axis=1), 1.0, atol=1e-12)


def pin_topk_special_rows(impl):
    nan, inf = np.nan, np.inf
    x = np.array([[1.0, nan, 5.0, nan, 2.0],
                  [-inf, -inf, -inf, -inf, -inf],
                  [0.0, inf, 1.0, inf, -2.0]], dtype=np.float32)
    tok, lp = impl.draft_topk(x, 3)
    assert list(tok[0]) == [1, 3, 2] and np.isnan(lp[0]).all()
    assert list(tok[1]) == [0, 1, 2] and (lp[1] == -inf).all()
    assert list(tok[2]) == [1, 3, 2] and np.isnan(lp[2]).all()


ALL_PINS = [pin_builder_is_global_order, pin_builder_limits, pin_topk_is_stable_sort, pin_topk_logp_closed_forms,
            pin_topk_special_rows]


def golden_ddtree_example():
    """The hand-worked builder example under tests/golden/."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "ddtree_worked_example.json")) as f:
        return json.load(f)


def pin_hand_worked_builder(impl):
    """The builder on the hand-worked example: parents and tokens id for id."""
    ex = golden_ddtree_example()
    par, tok = impl.build_tree(ex["root_token"], np.array(ex["tokens"], np.int32),
                               np.array(ex["logp"], np.float32), ex["budget"], ex["max_depth"])[:2]
    assert list(map(int, par)) == ex["parent"] and list(map(int, tok)) == ex["node_token"]


ALL_PINS.append(pin_hand_worked_builder)

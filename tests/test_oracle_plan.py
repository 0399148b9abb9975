"""Tree verdicts and traversal metadata of the oracle (CPU only)."""
import itertools

import numpy as np
import pytest

import workloads as W
from oracle import plan as P


def _simulate(parent, meta):
    """Follow the action words with symbolic states; every node must see its
    parent's state, the stack must never underflow and must end empty."""
    par = [int(p) for p in parent]
    cur, stack, seen = None, [], []
    for pos, x in enumerate(meta["order"]):
        act = int(meta["action"][pos])
        kind = act & 3
        if kind == P.ACT_INIT:
            assert par[x] == -1
            cur = "S0"
        elif kind == P.ACT_CONTINUE:
            assert cur == par[x]
        elif kind == P.ACT_TOP:
            assert stack and stack[-1] == par[x]
            cur = stack[-1]
        else:
            assert stack and stack[-1] == par[x]
            cur = stack.pop()
        seen.append(int(x))
        n_children = sum(1 for p in par if p == x)
        assert bool(act & P.ACT_LEAF) == (n_children == 0)
        assert bool(act & P.ACT_PUSH) == (n_children >= 2)
        if not act & P.ACT_LEAF:
            cur = int(x)
            if act & P.ACT_PUSH:
                stack.append(int(x))
    assert not stack
    assert sorted(seen) == list(range(len(par)))


def _check_preorder(parent, meta):
    par = [int(p) for p in parent]
    n = len(par)
    order = [int(x) for x in meta["order"]]
    pos = {x: i for i, x in enumerate(order)}
    size = meta["size"]
    for x in range(n):
        # a subtree occupies a contiguous run starting at its root
        desc = [y for y in range(n) if x in _path(par, y)]
        assert sorted(pos[y] for y in desc) == list(range(pos[x], pos[x] + len(desc)))
        assert size[x] == len(desc)
        kids = [c for c in range(n) if par[c] == x]
        visit = sorted(kids, key=lambda c: pos[c])
        assert visit == sorted(kids, key=lambda c: (size[c], c))


def _path(par, i):
    out = []
    while i != -1:
        out.append(i)
        i = par[i]
    return out


def test_metadata_exhaustive_small_trees():
    for choice in itertools.product(*[range(i) for i in range(1, 7)]):
        parent = np.array((-1,) + choice, dtype=np.int32)
        meta = P.plan_tree(parent)
        _simulate(parent, meta)
        _check_preorder(parent, meta)
        assert meta["max_stack"] <= P.stack_bound(7)
        for i in range(7):
            path = _path([int(p) for p in parent], i)[::-1]
            assert meta["depth"][i] == len(path)
            assert list(meta["nodepath"][i][: len(path)]) == path
            assert all(meta["nodepath"][i][len(path):] == -1)


@pytest.mark.parametrize("name", ["tiny", "chain", "ddtree22", "batched", "stress"])
def test_metadata_config_trees(name):
    cfg = W.get_config(name)
    for parent in W.make_trees(cfg)[:16]:
        meta = P.plan_tree(parent)
        _simulate(parent, meta)
        _check_preorder(parent, meta)
        assert meta["max_stack"] <= P.stack_bound(len(parent))


def test_forest_and_relabeled():
    rng = np.random.default_rng(3)
    parent = np.array([-1, 0, -1, 2, 2, -1, 1], dtype=np.int32)
    _simulate(parent, P.plan_tree(parent))
    for _ in range(20):
        base = W.random_tree(rng, 12, 5)
        perm = rng.permutation(12)
        _simulate(W.relabel(base, perm), P.plan_tree(W.relabel(base, perm)))


def test_stack_bound_is_tight():
    # complete binary trees reach the bound
    for levels in range(1, 7):
        n = 2 ** levels - 1
        parent = np.array([-1] + [(i - 1) // 2 for i in range(1, n)], dtype=np.int32)
        meta = P.plan_tree(parent)
        assert meta["max_stack"] == P.stack_bound(n) == levels - 1


def test_validate_verdicts():
    V = P.validate
    ok = np.array([-1, 0, 0, 1], np.int32)
    assert list(V(ok, [0, 4], [0], 1, 8, 16)) == [P.SEQ_OK]
    assert list(V(np.array([-1, 5, 0, 1], np.int32), [0, 4], [0], 1, 8, 16)) == [P.SEQ_BAD_PARENT]
    assert list(V(np.array([-1, 1, 0, 1], np.int32), [0, 4], [0], 1, 8, 16)) == [P.SEQ_BAD_PARENT]
    assert list(V(np.array([2, 0, 1, 1], np.int32), [0, 4], [0], 1, 8, 16)) == [P.SEQ_CYCLE_OR_DEPTH]
    chain = np.arange(-1, 17, dtype=np.int32)
    assert list(V(chain[:17], [0, 17], [0], 1, 32, 16)) == [P.SEQ_CYCLE_OR_DEPTH]
    assert list(V(chain[:16], [0, 16], [0], 1, 32, 16)) == [P.SEQ_OK]
    assert list(V(ok, [0, 4], [0], 1, 3, 16)) == [P.SEQ_BAD_NODES]
    assert list(V(ok, [0, 4], [1], 1, 8, 16)) == [P.SEQ_BAD_SLOT]
    two = np.concatenate([ok, ok])
    assert list(V(two, [0, 4, 8], [0, 0], 2, 8, 16)) == [P.SEQ_DUP_SLOT, P.SEQ_DUP_SLOT]
    # an empty sequence is inactive: its slot is neither checked nor counted
    assert list(V(ok, [0, 4, 4], [0, 0], 2, 8, 16)) == [P.SEQ_OK, P.SEQ_OK]
    assert list(V(ok, [0, 4, 4], [0, 99], 2, 8, 16)) == [P.SEQ_OK, P.SEQ_OK]
    assert list(V(ok, [0, 5], [0], 1, 8, 16)) == [P.SEQ_BAD_NODES]
    assert list(V(ok, [2, 1, 4], [0, 1], 2, 8, 16))[0] == P.SEQ_BAD_NODES


def test_hand_worked_example():
    """The traversal metadata worked by hand (tests/golden/plan_worked_example.json)."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "plan_worked_example.json")) as f:
        ex = json.load(f)
    r = P.plan_tree(np.array(ex["parent"], np.int32))
    assert np.asarray(r["depth"]).tolist() == ex["depth"]
    assert np.asarray(r["size"]).tolist() == ex["subtree_size"]
    assert np.asarray(r["order"]).tolist() == ex["order"]
    assert np.asarray(r["action"]).tolist() == ex["action"]
    m = ex["accepted_node"]
    assert [x for x in np.asarray(r["nodepath"])[m].tolist() if x >= 0] == ex["path"]

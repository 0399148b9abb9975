"""Pins of the fp64 oracle against facts fixed by the mathematics of the
gated delta rule and of tree traversal, independent of the oracle's own code.

Each ``pin_*`` function raises AssertionError when the oracle breaks the fact
it checks.  ``tests/test_oracle_pins.py`` runs them against the real oracle;
``tests/test_oracle_mutants.py`` runs them against copies of the oracle with a
planted mistake and expects every copy to fail at least one pin.

The rule:  S' = a S (I - b k k^T) + b v k^T,  o = S' q  (state D_v x D_k).
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle
from oracle.literal import literal_rule, path_replay, path_of

TINY_PARENT = np.array([-1, 0, 0, 1, 1, 2, 4], dtype=np.int32)


def golden_example():
    """The hand-worked 2x2 root-and-child example stored under tests/golden/."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "rule_2x2_worked_example.json")) as f:
        return json.load(f)


def unit(rng, *shape):
    g = rng.standard_normal(shape)
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def rand_case(rng, n, hk=2, hv=2, d=8, S_scale=1.0):
    return dict(
        q=unit(rng, n, hk, d), k=unit(rng, n, hk, d), v=rng.standard_normal((n, hv, d)),
        a=rng.uniform(0.2, 1.0, (n, hv)), b=rng.uniform(0.05, 1.0, (n, hv)),
        S0=S_scale * rng.standard_normal((hv, d, d)),
    )


def rel(x, r):
    m = np.abs(r).max()
    return np.abs(x - r).max() / (m if m > 0 else 1.0)


def run_tree(parent, c, states=False):
    return oracle.tree(parent, c["q"], c["k"], c["v"], c["a"], c["b"], c["S0"], return_states=states)


# ---------------------------------------------------------------- pins
def pin_tiny_unrolled():
    """The 7-node tree [-1,0,0,1,1,2,4], every node written out by hand with
    the literal matrix product (GQA 3:1 so value head h reads key head h//3)."""
    rng = np.random.default_rng(11)
    c = rand_case(rng, 7, hk=1, hv=3, d=6)
    out, st = run_tree(TINY_PARENT, c, states=True)
    for h in range(3):
        F = lambda S, j: literal_rule(S, c["k"][j, 0], c["v"][j, h], c["a"][j, h], c["b"][j, h])  # noqa: E731
        S = {}
        S[0] = F(c["S0"][h], 0)
        S[1] = F(S[0], 1)
        S[2] = F(S[0], 2)
        S[3] = F(S[1], 3)
        S[4] = F(S[1], 4)
        S[5] = F(S[2], 5)
        S[6] = F(S[4], 6)
        for j in range(7):
            assert rel(st[j, h], S[j]) < 1e-12, ("state", j, h)
            assert rel(out[j, h], S[j] @ c["q"][j, 0]) < 1e-12, ("out", j, h)


def pin_brute_force_small_trees(d=4, limit=None):
    """Every labeled 7-node tree with parent[i] < i (6! = 720 of them), kept
    when depth <= 4: the tree routine equals an independent per-node path
    replay with the literal rule."""
    rng = np.random.default_rng(12)
    c = rand_case(rng, 7, hk=1, hv=2, d=d)
    checked = 0
    for choice in itertools.product(*[range(i) for i in range(1, 7)]):
        parent = np.array((-1,) + choice, dtype=np.int32)
        depth = [len(path_of(parent, i)) for i in range(7)]
        if max(depth) > 4:
            continue
        out = run_tree(parent, c)
        for i in range(7):
            for h in range(2):
                S = path_replay(parent, i, c["S0"][h], c["k"][:, 0], c["v"][:, h], c["a"][:, h], c["b"][:, h])
                assert rel(out[i, h], S @ c["q"][i, 0]) < 1e-12, (choice, i, h)
        checked += 1
        if limit and checked >= limit:
            break
    return checked


def pin_closed_forms():
    rng = np.random.default_rng(13)
    n, d = 6, 8
    parent = np.array([-1, 0, 1, 1, 3, 0], dtype=np.int32)
    # (1) b = 0: pure decay, S^n = (prod of a on the path) S0
    c = rand_case(rng, n, d=d)
    c["b"][:] = 0.0
    out = run_tree(parent, c)
    for i in range(n):
        for h in range(2):
            g = np.prod([c["a"][j, h] for j in path_of(parent, i)])
            assert rel(out[i, h], g * c["S0"][h] @ c["q"][i, h]) < 1e-13, ("decay", i, h)
    # (2) a = 1, b = 0: the state never changes
    c["a"][:] = 1.0
    out = run_tree(parent, c)
    for i in range(n):
        for h in range(2):
            assert rel(out[i, h], c["S0"][h] @ c["q"][i, h]) < 1e-13
    # (3) zero state, single node: o = b (k . q) v
    c = rand_case(rng, 1, d=d)
    c["S0"][:] = 0.0
    out = run_tree(np.array([-1], np.int32), c)
    for h in range(2):
        ref = c["b"][0, h] * (c["k"][0, h] @ c["q"][0, h]) * c["v"][0, h]
        assert rel(out[0, h], ref) < 1e-13
    # (4) retrieval: with b = 1 and |k| = 1, S' k = v whatever S and a are
    c = rand_case(rng, n, d=d)
    c["b"][:] = 1.0
    c["q"] = c["k"].copy()
    out = run_tree(parent, c)
    for i in range(n):
        for h in range(2):
            assert rel(out[i, h], c["v"][i, h]) < 1e-12, ("retrieval", i, h)
    # (5) a = 1: S' k = (1 - b) S k + b v  (|k| = 1), read at the parent state
    c = rand_case(rng, n, d=d)
    c["a"][:] = 1.0
    c["q"] = c["k"].copy()
    out, st = run_tree(parent, c, states=True)
    for i in range(n):
        for h in range(2):
            p = parent[i]
            Sp = c["S0"][h] if p < 0 else st[p, h]
            bb = c["b"][i, h]
            ref = (1 - bb) * Sp @ c["k"][i, h] + bb * c["v"][i, h]
            assert rel(out[i, h], ref) < 1e-12
    # (6) directions orthogonal to k only decay: S' x = a S x for x . k = 0
    c = rand_case(rng, n, d=d)
    out, st = run_tree(parent, c, states=True)
    for i in range(n):
        for h in range(2):
            k = c["k"][i, h]
            x = rng.standard_normal(d)
            x -= (x @ k) * k
            p = parent[i]
            Sp = c["S0"][h] if p < 0 else st[p, h]
            assert rel(st[i, h] @ x, c["a"][i, h] * Sp @ x) < 1e-12


def pin_chain_equals_sequential():
    """A chain tree (W = 1) gives the sequential recurrence's outputs."""
    rng = np.random.default_rng(14)
    L = 16
    c = rand_case(rng, L, hk=2, hv=6, d=8)
    par = np.arange(-1, L - 1, dtype=np.int32)
    out_t, st = run_tree(par, c, states=True)
    out_c, fin = oracle.chain(c["k"], c["v"], c["a"], c["b"], c["S0"], q=c["q"])
    assert rel(out_t, out_c) < 1e-12
    assert rel(st[-1], fin) < 1e-12
    # and the sequential recurrence itself, unrolled with the literal rule
    for h in range(6):
        S = c["S0"][h]
        for t in range(L):
            S = literal_rule(S, c["k"][t, h // 3], c["v"][t, h], c["a"][t, h], c["b"][t, h])
            assert rel(out_c[t, h], S @ c["q"][t, h // 3]) < 1e-12


def pin_superposition():
    """The rule is linear in (S, v): o(S0 + S0', v + v') = o(S0, v) + o(S0', v')."""
    rng = np.random.default_rng(15)
    parent = np.array([-1, 0, 0, 1, 2, 2, 5, 0], dtype=np.int32)
    c1 = rand_case(rng, 8, d=8)
    c2 = dict(c1, v=rng.standard_normal(c1["v"].shape), S0=rng.standard_normal(c1["S0"].shape))
    c12 = dict(c1, v=c1["v"] + c2["v"], S0=c1["S0"] + c2["S0"])
    o1, o2, o12 = run_tree(parent, c1), run_tree(parent, c2), run_tree(parent, c12)
    assert rel(o12, o1 + o2) < 1e-12


def pin_duplicate_siblings():
    """Two identical sibling subtrees (same inputs) give identical outputs."""
    rng = np.random.default_rng(16)
    # root 0; subtree A = 1 -> 3 -> 5, subtree B = 2 -> 4 -> 6 mirrors A
    parent = np.array([-1, 0, 0, 1, 2, 3, 4], dtype=np.int32)
    c = rand_case(rng, 7, d=8)
    for x in ("q", "k", "v", "a", "b"):
        for a_, b_ in ((1, 2), (3, 4), (5, 6)):
            c[x][b_] = c[x][a_]
    out = run_tree(parent, c)
    for a_, b_ in ((1, 2), (3, 4), (5, 6)):
        assert np.array_equal(out[a_], out[b_])
    assert not np.array_equal(out[1], out[3])


def pin_ancestor_only():
    """o_n depends only on the inputs of n's ancestors (and n)."""
    rng = np.random.default_rng(17)
    parent = np.array([-1, 0, 0, 1, 1, 2, 4, 3], dtype=np.int32)
    c = rand_case(rng, 8, d=8)
    out = run_tree(parent, c)
    for target in range(8):
        anc = set(path_of(parent, target))
        c2 = {x: c[x].copy() for x in c}
        for j in range(8):
            if j not in anc:
                for x in ("q", "k", "v", "a", "b"):
                    c2[x][j] = c2[x][j] * 0.5 + 0.1
        out2 = run_tree(parent, c2)
        assert np.array_equal(out2[target], out[target])
        changed = [j for j in range(8) if j not in anc and not np.array_equal(out2[j], out[j])]
        assert changed == [j for j in range(8) if j not in anc]


def pin_permutation():
    """Relabeling nodes permutes outputs; permuting value rows permutes o."""
    rng = np.random.default_rng(18)
    parent = np.array([-1, 0, 1, 0, 3, 3, 2, 6, 4], dtype=np.int32)
    n = len(parent)
    c = rand_case(rng, n, d=8)
    out = run_tree(parent, c)
    perm = rng.permutation(n)
    inv = np.argsort(perm)
    new_parent = np.array([-1 if parent[inv[i]] < 0 else perm[parent[inv[i]]] for i in range(n)], np.int32)
    c2 = {x: (c[x][inv] if x != "S0" else c[x]) for x in c}
    out2 = run_tree(new_parent, c2)
    assert np.array_equal(out2[perm], out)
    rows = rng.permutation(8)
    c3 = dict(c, v=c["v"][:, :, rows], S0=c["S0"][:, rows, :])
    out3 = run_tree(parent, c3)
    assert np.array_equal(out3, out[:, :, rows])


def pin_persist_replay():
    """The accepted node's state equals the state the tree routine stored for
    it, and equals a literal replay of the root-to-node path."""
    rng = np.random.default_rng(19)
    parent = np.array([-1, 0, 0, 1, 1, 2, 4, 6, 6], dtype=np.int32)
    c = rand_case(rng, 9, hk=1, hv=3, d=8)
    _, st = run_tree(parent, c, states=True)
    for m in range(9):
        S, path = oracle.accept_state(parent, m, c["k"], c["v"], c["a"], c["b"], c["S0"])
        assert list(path) == path_of(parent, m)
        assert np.array_equal(S, st[m])
        for h in range(3):
            ref = path_replay(parent, m, c["S0"][h], c["k"][:, 0], c["v"][:, h], c["a"][:, h], c["b"][:, h])
            assert rel(S[h], ref) < 1e-12


def pin_forest():
    """Several roots: each root starts from the committed state."""
    rng = np.random.default_rng(20)
    parent = np.array([-1, 0, -1, 2, -1], dtype=np.int32)
    c = rand_case(rng, 5, d=8)
    out = run_tree(parent, c)
    for i in range(5):
        for h in range(2):
            S = path_replay(parent, i, c["S0"][h], c["k"][:, h], c["v"][:, h], c["a"][:, h], c["b"][:, h])
            assert rel(out[i, h], S @ c["q"][i, h]) < 1e-12


def pin_batch_wrappers():
    """verify_batch and persist_batch, which give every multi-sequence GPU test its
    expected values: each sequence's node state is the rule over its own
    root-to-node path from its own committed state (magik.net page, "The Broader
    Context"; GreenGames page, "From autoregressive to DDTree").  Checked node by
    node against the literal per-path replay on a ragged batch: sizes 5, 0, 7 (a
    forest of three roots), 1 and 4; a distinct committed state per sequence;
    value head h reading key head h // 2; one sequence skipped (accepted -1)."""
    rng = np.random.default_rng(21)
    trees = [np.array([-1, 0, 0, 1, 3], np.int32), np.zeros(0, np.int32),
             np.array([-1, 0, -1, 2, -1, 4, 5], np.int32), np.array([-1], np.int32),
             np.array([-1, 0, 1, 1], np.int32)]
    sizes = [len(t) for t in trees]
    cu = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    T, hk, hv, d = int(cu[-1]), 2, 4, 5
    inputs = dict(q=unit(rng, T, hk, d), k=unit(rng, T, hk, d), v=rng.standard_normal((T, hv, d)),
                  a=rng.uniform(0.2, 1.0, (T, hv)), b=rng.uniform(0.05, 1.0, (T, hv)))
    S0_seq = rng.standard_normal((len(trees), hv, d, d))
    accepted = np.array([4, -1, 6, 0, -1], np.int32)
    accepted[4] = -1  # a non-empty sequence skipped
    out = oracle.verify_batch(trees, cu, inputs, S0_seq)
    res = oracle.persist_batch(trees, cu, inputs, S0_seq, accepted)
    assert out.shape == (T, hv, d) and len(res) == len(trees)
    for s, par in enumerate(trees):
        lo = int(cu[s])
        for i in range(len(par)):
            for h in range(hv):
                g = h // (hv // hk)
                sl = slice(lo, lo + len(par))
                S = path_replay(par, i, S0_seq[s][h], inputs["k"][sl, g], inputs["v"][sl, h], inputs["a"][sl, h],
                                inputs["b"][sl, h])
                assert rel(out[lo + i, h], S @ inputs["q"][lo + i, g]) < 1e-12, (s, i, h)
        st, path = res[s]
        m = int(accepted[s])
        if m < 0 or len(par) == 0:
            assert st is None and len(path) == 0, s
            continue
        assert list(path) == path_of(par, m), s
        for h in range(hv):
            g = h // (hv // hk)
            sl = slice(lo, lo + len(par))
            S = path_replay(par, m, S0_seq[s][h], inputs["k"][sl, g], inputs["v"][sl, h], inputs["a"][sl, h],
                            inputs["b"][sl, h])
            assert rel(st[h], S) < 1e-12, (s, h)


ALL_PINS = [
    pin_tiny_unrolled, pin_closed_forms, pin_chain_equals_sequential, pin_superposition,
    pin_duplicate_siblings, pin_ancestor_only, pin_permutation, pin_persist_replay, pin_forest,
    pin_batch_wrappers, lambda: pin_brute_force_small_trees(limit=60),
]

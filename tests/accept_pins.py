"""Pins of the greedy-acceptance oracle (``oracle/accept.py``) against facts
that do not depend on its code.

Each ``pin_*(impl)`` takes a module with the oracle's ``accept`` and
``target_tokens`` functions and raises AssertionError when it breaks the fact
it checks.  ``tests/test_oracle_accept.py`` runs them on the real oracle and on
copies of it with a planted mistake (each copy must fail at least one pin).

The central fact: at temperature 0 a lossless speculative decoder emits the
tokens plain autoregressive greedy decoding emits
(dflash-caddtree-integrations README, "The shared method").  The pins build a
deterministic toy "target model" -- a hash from the context tokens to the next
token -- decode it autoregressively, and require the accepted path to be the
longest tree path that spells out a prefix of that decode, and the next token
to be the decode's following token.
"""
from __future__ import annotations

import numpy as np

SEQ_OK = 0


def toy_next(ctx: tuple, vocab: int) -> int:
    """Deterministic next token for a context (an arbitrary fixed hash)."""
    h = 1469598103
    for t in ctx:
        h = ((h ^ (int(t) + 7)) * 1099511) % 2305843009213693951
    return int(h % vocab)


def path_to(parent, n):
    p = []
    while n != -1:
        p.append(n)
        n = int(parent[n])
    return p[::-1]


def build_case(rng, parent, vocab, prefix=(3, 1, 4), p_follow=0.6):
    """Draft tokens (distinct among siblings) where a child follows the toy
    target with probability ``p_follow``, and logits whose argmax in row u is
    the toy target's prediction after u's context."""
    n = len(parent)
    tok = np.zeros(n, dtype=np.int64)
    tok[[i for i in range(n) if parent[i] == -1]] = prefix[-1]
    ctx_of = {}
    for u in range(n):  # parents precede children in these trees
        if parent[u] == -1:
            ctx_of[u] = tuple(prefix)
    kids = [[c for c in range(n) if parent[c] == u] for u in range(n)]
    for u in range(n):
        want = toy_next(ctx_of[u], vocab)
        used = set()
        for c in kids[u]:
            if rng.random() < p_follow and want not in used:
                t = want
            else:
                t = int(rng.integers(vocab))
                while t in used or t == want:
                    t = int(rng.integers(vocab))
            used.add(t)
            tok[c] = t
            ctx_of[c] = ctx_of[u] + (t,)
    logits = rng.standard_normal((n, vocab)).astype(np.float32)
    for u in range(n):
        logits[u, toy_next(ctx_of[u], vocab)] = 50.0
    return tok, logits, ctx_of


def ar_expectation(parent, tok, prefix, vocab, max_len):
    """Autoregressive greedy decode, then the deepest node whose path spells
    a prefix of it (brute force over every node)."""
    ctx = tuple(prefix)
    ar = []
    for _ in range(max_len + 1):
        t = toy_next(ctx, vocab)
        ar.append(t)
        ctx = ctx + (t,)
    best, best_len = None, 0
    roots = [i for i in range(len(parent)) if parent[i] == -1]
    for u in range(len(parent)):
        p = path_to(parent, u)
        if p[0] != min(roots):
            continue
        spelled = [int(tok[x]) for x in p[1:]]
        if spelled == ar[: len(spelled)] and len(p) > best_len:
            best, best_len = u, len(p)
    return best, best_len, ar[best_len - 1]


def random_parent(rng, n, width):
    par = [-1]
    nk = [0]
    for i in range(1, n):
        cand = [j for j in range(i) if nk[j] < width]
        p = cand[int(rng.integers(len(cand)))]
        par.append(p)
        nk[p] += 1
        nk.append(0)
    return np.array(par, dtype=np.int64)


def pin_autoregressive_equivalence(impl):
    rng = np.random.default_rng(11)
    vocab = 97
    for trial in range(60):
        n = int(rng.integers(1, 24))
        par = random_parent(rng, n, int(rng.integers(1, 5)))
        prefix = tuple(int(x) for x in rng.integers(0, vocab, 3))
        tok, logits, _ = build_case(rng, par, vocab, prefix, p_follow=float(rng.uniform(0.3, 0.95)))
        exp_node, exp_len, exp_next = ar_expectation(par, tok, prefix, vocab, n)
        acc, alen, nxt, _ = impl.accept(par, np.array([0, n]), tok, logits, np.array([SEQ_OK]))
        assert (acc[0], alen[0], nxt[0]) == (exp_node, exp_len, exp_next), (trial, acc, alen, nxt, exp_node, exp_len, exp_next)


def pin_chain_prefix_length(impl):
    """A chain whose drafts agree with the target for exactly j steps
    accepts j + 1 nodes and ends at node j."""
    vocab = 50
    n = 9
    par = np.arange(-1, n - 1)
    for j in range(n):
        logits = np.zeros((n, vocab), dtype=np.float32)
        tok = np.zeros(n, dtype=np.int64)
        for u in range(n):
            logits[u, (5 * u + 2) % vocab] = 1.0
        for c in range(1, n):
            want = (5 * (c - 1) + 2) % vocab
            tok[c] = want if c <= j else (want + 1) % vocab
        acc, alen, nxt, _ = impl.accept(par, np.array([0, n]), tok, logits, np.array([SEQ_OK]))
        assert acc[0] == j and alen[0] == j + 1 and nxt[0] == (5 * j + 2) % vocab, (j, acc, alen, nxt)


def pin_argmax_special_values(impl):
    """First-index rule for equal values (+0 equals -0), NaN counts as the
    largest value, an all -inf row gives index 0 (values written by hand)."""
    nan, inf = np.nan, np.inf
    rows = [
        ([1.0, 3.0, 3.0, 2.0], 1),
        ([-0.0, 0.0, -1.0], 0),
        ([0.0, -0.0, -1.0], 0),
        ([1.0, nan, 5.0, nan], 1),
        ([-inf, -inf, -inf], 0),
        ([-inf, -3e38, -inf], 1),
        ([inf, 1.0, inf], 0),
        ([-1.0, -2.0, -0.5, -0.5], 2),
        ([7.0], 0),
    ]
    for vals, want in rows:
        got = impl.target_tokens(np.array([vals], dtype=np.float32))
        assert got[0] == want, (vals, got, want)


def pin_forest_and_duplicates(impl):
    """Readings: a forest starts at its smallest root; equal sibling tokens
    resolve to the smaller child id; other roots are never accepted."""
    vocab = 10
    # roots 1 and 3; node 2 (child of 1) and node 0 (child of 3)
    par = np.array([3, -1, 1, -1])
    logits = np.zeros((4, vocab), dtype=np.float32)
    logits[1, 6] = 1.0
    logits[2, 4] = 1.0
    logits[3, 6] = 1.0
    tok = np.array([6, 0, 6, 0])
    acc, alen, nxt, _ = impl.accept(par, np.array([0, 4]), tok, logits, np.array([SEQ_OK]))
    assert (acc[0], alen[0], nxt[0]) == (2, 2, 4)
    # two children with the same (matching) token: the smaller id wins
    par = np.array([-1, 0, 0, 2])
    tok = np.array([0, 5, 5, 8])
    logits = np.zeros((4, vocab), dtype=np.float32)
    logits[0, 5] = 1.0
    logits[2, 8] = 1.0
    logits[1, 9] = 1.0
    acc, alen, nxt, _ = impl.accept(par, np.array([0, 4]), tok, logits, np.array([SEQ_OK]))
    assert (acc[0], alen[0], nxt[0]) == (1, 2, 9)


def pin_rejected_and_empty(impl):
    vocab = 6
    par = np.array([-1, 0, -1])
    cu = np.array([0, 2, 2, 3])
    tok = np.array([0, 1, 0])
    logits = np.zeros((3, vocab), dtype=np.float32)
    logits[0, 1] = 1.0
    acc, alen, nxt, tgt = impl.accept(par, cu, tok, logits, np.array([SEQ_OK, SEQ_OK, 4]))
    assert list(acc) == [1, -1, -1] and list(alen) == [2, 0, 0] and list(nxt) == [0, -1, -1]
    assert list(tgt) == [1, 0, 0]


def pin_hand_worked(impl):
    """The hand-worked example under tests/golden/."""
    ex, logits = golden_accept_example()
    got = impl.accept(np.array(ex["parent"], np.int32), np.array(ex["cu_nodes"]),
                      np.array(ex["draft_token"], np.int32), logits, np.zeros(len(ex["cu_nodes"]) - 1, np.int32))
    for g, key in zip(got, ("accepted_node", "accept_len", "next_token", "target")):
        assert np.array_equal(g, ex[key]), key


ALL_PINS = [pin_autoregressive_equivalence, pin_chain_prefix_length, pin_argmax_special_values,
            pin_forest_and_duplicates, pin_rejected_and_empty, pin_hand_worked]


def golden_accept_example():
    """The hand-worked acceptance example under tests/golden/: its inputs (logits
    rebuilt from the stated background, entries and NaNs) and the hand-derived
    results."""
    import json
    import os
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                           "accept_worked_example.json")) as f:
        ex = json.load(f)
    V, T = ex["vocab"], len(ex["parent"])
    logits = np.tile(-1.0 - np.arange(V) / 16.0, (T, 1)).astype(np.float32)
    for r, c, v in ex["set"]:
        logits[r, c] = v
    for r, c in ex["nan_at"]:
        logits[r, c] = np.nan
    return ex, logits

"""Greedy (temperature-0) acceptance of draft trees against the target's verify logits.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What it computes.  One target forward over a draft tree yields a logits row
per node: the target's prediction for the token that follows that node on its
root-to-node path (the GreenGames page, "Key wins": the verify logits buffer
holds one vocabulary-wide row per tree node, budget + 1 rows).  Verification
there is greedy only ("What comes next"), and a lossless speculative decoder
must emit exactly the tokens plain autoregressive decoding would at
temperature 0 (dflash-caddtree-integrations README, "The shared method").  So:

  target[n]  = the first index of the largest value of row n (numpy argmax:
               a NaN counts as the largest value, equal values keep the first)
  walk       = start at the sequence's root (the smallest local id among the
               roots of a forest); while some child c of the current node u
               carries draft_token[c] == target[u], move to the smallest such c
  accepted   = the node where the walk stops; accept_len = its depth (root = 1);
  next_token = target[accepted] (the token the target emits after the path).

A rejected or empty sequence yields accepted = -1, accept_len = 0 and
next_token = -1.  The root's own draft token is never compared (it is the
already committed token).
"""
from __future__ import annotations

import numpy as np

from .plan import SEQ_OK


def target_tokens(logits: np.ndarray) -> np.ndarray:
    """Row-wise argmax of [T][V] logits (numpy's first-NaN / first-max rule)."""
    logits = np.asarray(logits)
    if logits.shape[0] == 0:
        return np.zeros(0, dtype=np.int32)
    return np.argmax(logits, axis=1).astype(np.int32)


def accept_one(parent: np.ndarray, draft_token: np.ndarray, target: np.ndarray):
    """Greedy walk over one valid, non-empty tree.  Returns (node, length)."""
    n = len(parent)
    cur = min(i for i in range(n) if parent[i] == -1)
    length = 1
    while True:
        want = int(target[cur])
        kids = [c for c in range(n) if parent[c] == cur and int(draft_token[c]) == want]
        if not kids:
            return cur, length
        cur = min(kids)
        length += 1


def accept(parent, cu_nodes, draft_token, logits, status):
    """All sequences.  ``status`` holds the plan's verdict per sequence.

    Returns (accepted_node [B], accept_len [B], next_token [B], target [T]) int32."""
    parent = np.asarray(parent, dtype=np.int64)
    draft_token = np.asarray(draft_token, dtype=np.int64)
    cu = np.asarray(cu_nodes, dtype=np.int64)
    target = target_tokens(logits)
    nseq = len(cu) - 1
    acc = np.full(nseq, -1, dtype=np.int32)
    alen = np.zeros(nseq, dtype=np.int32)
    nxt = np.full(nseq, -1, dtype=np.int32)
    for s in range(nseq):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if int(status[s]) != SEQ_OK or hi <= lo:
            continue
        node, length = accept_one(parent[lo:hi], draft_token[lo:hi], target[lo:hi])
        acc[s], alen[s], nxt[s] = node, length, target[lo + node]
    return acc, alen, nxt, target

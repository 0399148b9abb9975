"""Draft-tree generators (parent-pointer form, local node ids, -1 = root).

The DDTree generator stands in for the DFlash drafter + ``build_ddtree`` of the
GreenGames page (section "From autoregressive to DDTree": a chain pre-seed;
section "Key wins": candidates ranked in descending order, best first).  The
pages give no scoring rule, so the tree is grown best-first under factorized
per-level top-W probabilities: a candidate's score is the sum of log
probabilities along its path.  Node ids follow insertion order, so every
parent id is smaller than its child's.
"""
from __future__ import annotations

import heapq

import numpy as np


def chain_tree(n: int) -> np.ndarray:
    """parent[i] = i - 1: the W=1 linear block."""
    return np.arange(-1, n - 1, dtype=np.int32)


def random_tree(rng: np.random.Generator, n: int, max_depth: int) -> np.ndarray:
    """Node i > 0 picks its parent uniformly among earlier nodes of depth < max_depth."""
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int64)
    if n == 0:
        return parent
    depth[0] = 1
    for i in range(1, n):
        cand = [j for j in range(i) if depth[j] < max_depth]
        p = cand[int(rng.integers(len(cand)))]
        parent[i] = p
        depth[i] = depth[p] + 1
    return parent


def ddtree_tree(rng: np.random.Generator, budget: int, width: int, dmax: int) -> np.ndarray:
    """Best-first top-W tree of ``budget`` drafts below a root (budget + 1 nodes).

    1. For each draft level l = 1 .. dmax-1 draw ``width`` logits ~ N(0, 2^2),
       softmax them and sort descending (rank 1 is the most likely token).
    2. Chain pre-seed: nodes 1 .. min(budget, dmax-1) form the rank-1 chain.
    3. Fill best-first by path score (sum of log p) with <= width children per
       node and depth <= dmax, until there are ``budget`` drafts.
       Ties: higher score, then smaller depth, then smaller rank, then smaller
       parent id.
    """
    levels = dmax - 1
    logp = np.empty((levels + 1, width), dtype=np.float64)
    logp[0] = 0.0
    for lvl in range(1, levels + 1):
        z = rng.normal(0.0, 2.0, size=width)
        z = z - z.max()
        p = np.exp(z) / np.exp(z).sum()
        logp[lvl] = np.log(np.sort(p)[::-1])

    parent = [-1]
    depth = [1]
    score = [0.0]
    nchild = [0]

    def add(par: int) -> int:
        rank = nchild[par]
        nchild[par] += 1
        parent.append(par)
        depth.append(depth[par] + 1)
        score.append(score[par] + logp[depth[par]][rank])
        nchild.append(0)
        return len(parent) - 1

    # chain pre-seed along rank 1
    seed_len = min(budget, levels)
    cur = 0
    for _ in range(seed_len):
        cur = add(cur)

    heap: list = []

    def push_candidate(par: int) -> None:
        if depth[par] >= dmax or nchild[par] >= width:
            return
        rank = nchild[par]
        s = score[par] + logp[depth[par]][rank]
        heapq.heappush(heap, (-s, depth[par] + 1, rank, par))

    for node in range(len(parent)):
        push_candidate(node)
    while len(parent) - 1 < budget and heap:
        _, _, rank, par = heapq.heappop(heap)
        if nchild[par] != rank:  # stale entry (sibling already taken)
            continue
        child = add(par)
        push_candidate(par)
        push_candidate(child)
    return np.asarray(parent, dtype=np.int32)


def tree_depths(parent: np.ndarray) -> np.ndarray:
    """Depth of every node of a valid tree, root = 1 (index bookkeeping only)."""
    n = len(parent)
    depth = np.zeros(n, dtype=np.int32)
    for i in range(n):
        d, j = 0, i
        while j != -1:
            d += 1
            j = int(parent[j])
            if d > n:
                raise ValueError("cycle in parent array")
        depth[i] = d
    return depth


def relabel(parent: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Rename node i to perm[i]; returns the parent array of the renamed tree."""
    n = len(parent)
    new_parent = np.full(n, -1, dtype=np.int32)
    for i in range(n):
        p = int(parent[i])
        new_parent[perm[i]] = -1 if p < 0 else perm[p]
    return new_parent

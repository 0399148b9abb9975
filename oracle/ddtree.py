"""Draft top-k extraction and the DDTree tree builder, written out plainly.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

What it computes (GreenGames page, "From autoregressive to DDTree" and "Key
wins"; magik.net page, "The Broader Context").  The drafter scores every
vocabulary entry at each of the L positions of its block.  Per position the
builder keeps the W best candidates in descending order -- rank 1 first, the
order whose accidental reversal sent the worst candidate to the tree root --
with their log-probabilities, and grows a tree of ``budget`` drafts below the
root (the last committed token):

  top-k    candidates of a row in argmax order (a NaN counts as largest, equal
           values keep the smaller id); log p = x - logsumexp(row), in fp64
           (all NaN when the row holds a NaN or +inf, all -inf when every
           entry is -inf; ranks past the vocabulary get token -1, log p -inf).
  builder  1. chain pre-seed: nodes 1 .. min(budget, L) form the rank-1 chain;
           2. best first: a node at depth d (root = 1) may take its next
              unused rank r < W at level d (its child's position) while
              d < min(L + 1, max_depth); the candidate's score is the parent's
              score plus that level's log p of rank r, accumulated in fp32
              (NaN log p counts as -inf); the best candidate -- higher score,
              then smaller child depth, then smaller rank, then smaller parent
              id -- becomes the next node, until ``budget`` drafts exist or no
              candidate is left.
           Node ids follow insertion order, so every parent id is smaller than
           its child's; a node's token is its level's candidate of its rank.
"""
from __future__ import annotations

import heapq

import numpy as np

MAX_WIDTH = 16


def draft_topk(logits: np.ndarray, width: int):
    """Rows [R][V] -> (tokens [R][W] int32, log p [R][W] float64)."""
    logits = np.asarray(logits, dtype=np.float32)
    R, V = logits.shape
    w = min(width, V)
    toks = np.zeros((R, width), dtype=np.int32)
    logp = np.full((R, width), -np.inf)
    idx = np.arange(V)
    for r in range(R):
        x = logits[r].astype(np.float64)
        nan = np.isnan(x)
        # np.lexsort sorts by its last key first: NaNs, then larger values, then smaller ids
        order = np.lexsort((idx, -np.where(nan, 0.0, x), ~nan))
        toks[r, :w] = order[:w]
        m = x.max() if not nan.any() else np.nan
        if np.isnan(m) or m == np.inf:   # no distribution: a NaN, or an infinite logit
            logp[r, :w] = np.nan
        elif m == -np.inf:                # every candidate impossible
            logp[r, :w] = -np.inf
        else:
            logp[r, :w] = x[order[:w]] - (m + np.log(np.exp(x - m).sum()))
    if w < width:
        toks[:, w:] = -1
    return toks, logp


def tree_size(levels: int, width: int, budget: int, max_depth: int = 16) -> int:
    """Nodes of every built tree: the root plus min(budget, all nodes the
    depth and width limits allow)."""
    depth_cap = min(levels + 1, max_depth)
    cap, layer = 0, 1
    for _ in range(1, depth_cap):
        layer *= width
        cap += layer
        if cap >= budget:
            break
    return 1 + min(budget, cap)


def build_tree(root_token: int, tokens: np.ndarray, logp: np.ndarray, budget: int, max_depth: int = 16,
               margins: list | None = None):
    """One sequence.  tokens/logp [L][W] (level l = 1 .. L in row l - 1).
    Returns (parent, token, score) of the built tree, root first.  If a list is
    given as ``margins``, each best-first choice appends the score gap to the
    best other live candidate (inf when it had none)."""
    tokens = np.asarray(tokens)
    L, W = tokens.shape
    lp = np.asarray(logp, dtype=np.float32)
    lp = np.where(np.isnan(lp), np.float32(-np.inf), lp).astype(np.float32)
    depth_cap = min(L + 1, max_depth)

    parent = [-1]
    token = [int(root_token)]
    depth = [1]
    score = [np.float32(0.0)]
    nchild = [0]

    def add(par: int) -> int:
        r = nchild[par]
        nchild[par] += 1
        parent.append(par)
        token.append(int(tokens[depth[par] - 1, r]))
        depth.append(depth[par] + 1)
        score.append(np.float32(score[par] + lp[depth[par] - 1, r]))
        nchild.append(0)
        return len(parent) - 1

    # 1. the rank-1 chain
    cur = 0
    while len(parent) - 1 < budget and depth[cur] < depth_cap and W > 0:
        cur = add(cur)

    # 2. best first over every node's next unused rank
    heap: list = []

    def offer(par: int) -> None:
        if depth[par] >= depth_cap or nchild[par] >= W:
            return
        r = nchild[par]
        s = np.float32(score[par] + lp[depth[par] - 1, r])
        # heapq pops the smallest tuple: negated score (-inf scores sort last),
        # then child depth, rank and parent id ascending
        heapq.heappush(heap, (-float(s), depth[par] + 1, r, par))

    for node in range(len(parent)):
        offer(node)
    while len(parent) - 1 < budget and heap:
        neg, _, r, par = heapq.heappop(heap)
        if nchild[par] != r:
            continue
        if margins is not None:
            live = [-e[0] for e in heap if nchild[e[3]] == e[2]]
            margins.append(-neg - max(live) if live else np.inf)
        child = add(par)
        offer(par)
        offer(child)
    return (np.asarray(parent, dtype=np.int32), np.asarray(token, dtype=np.int32),
            np.asarray(score, dtype=np.float32))


def build_batch(root_tokens, tokens, logp, budget: int, max_depth: int = 16):
    """All sequences: tokens/logp [B][L][W].  Returns (parent [B*N], token [B*N],
    cu_nodes [B+1]) with every tree N = tree_size(...) nodes long."""
    tokens = np.asarray(tokens)
    B, L, W = tokens.shape
    N = tree_size(L, W, budget, max_depth)
    par = np.zeros(B * N, dtype=np.int32)
    tok = np.zeros(B * N, dtype=np.int32)
    for b in range(B):
        p, t, _ = build_tree(int(root_tokens[b]), tokens[b], logp[b], budget, max_depth)
        assert len(p) == N, (len(p), N)
        par[b * N:(b + 1) * N] = p
        tok[b * N:(b + 1) * N] = t
    cu = (np.arange(B + 1) * N).astype(np.int32)
    return par, tok, cu

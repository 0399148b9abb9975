"""Seeded draft tokens and target verify logits for greedy acceptance.

The pages print no vocabulary size; the workloads take V = 248,320, the size
of the Qwen3.5 tokenizer (the target family on the GreenGames page).  The
verify logits buffer holds one fp32 row of V entries per tree node (GreenGames
page, "Key wins": vocab x (budget + 1) rows).

Recipe.
  Draft tokens: DDTree's drafter proposes, per block position (tree level), a
  ranked list of candidate tokens, and a node at level l with sibling rank r
  carries candidate r of level l (GreenGames page, "Key wins": candidates in
  descending order).  Per sequence and level we draw ``width`` distinct
  tokens uniformly from [0, V); a node's rank is its position among its
  siblings by id (the generators insert rank 1 first), so siblings always
  carry distinct tokens.
  Logits: every row ~ N(0, 1) in float32.  Each node's row gets one planted
  entry of value ``planted`` at the token the target "prefers" there: the
  token of the node's rank-r child with probability ``match[r-1]``, else a
  uniform token that no child carries.  Leaves always get a uniform token.

  Draft logits (the drafter's scores over the vocabulary at each of the
  DRAFT_LEVELS = 15 drafted positions of a 16-token block, GreenGames
  "Prefill"): every row N(0, 1) in float32, plus ``width`` distinct uniform
  tokens planted at 20 + z with z ~ N(0, 2^2) -- the per-level candidate
  logits of the tree recipe, lifted far enough above the noise that the
  drafter's mass sits on them.  Root tokens: uniform in [0, V).

Streams: numpy PCG64 from ``SeedSequence(cfg.seed, spawn_key=(4|5|6|7, seq))``.
"""
from __future__ import annotations

import numpy as np

from .configs import Config
from .inputs import _rng

VOCAB = 248320
DRAFT_LEVELS = 15
_DRAFT, _LOGITS, _DLOGITS, _ROOT = 4, 5, 6, 7
MATCH = (0.7, 0.1, 0.05, 0.03)


def _children_by_rank(parent: np.ndarray) -> list[list[int]]:
    kids: list[list[int]] = [[] for _ in range(len(parent))]
    for c, p in enumerate(parent):
        if p >= 0:
            kids[int(p)].append(c)
    return kids


def _levels(parent: np.ndarray) -> np.ndarray:
    lvl = np.zeros(len(parent), dtype=np.int64)
    for i in range(len(parent)):
        d, j = 0, i
        while parent[j] != -1 and d <= len(parent):
            d += 1
            j = int(parent[j])
        lvl[i] = d
    return lvl


def make_draft_tokens(cfg: Config, trees: list[np.ndarray], vocab: int = VOCAB) -> np.ndarray:
    """int32 [T]: the draft token of every node (roots carry a token too; it is
    the committed token and never compared)."""
    out = []
    for s, par in enumerate(trees):
        n = len(par)
        rng = _rng(cfg, _DRAFT, s)
        kids = _children_by_rank(par)
        width = max([len(k) for k in kids] + [1])
        lvl = _levels(par)
        nlev = int(lvl.max()) + 1 if n else 1
        table = np.stack([rng.choice(vocab, size=min(width, vocab), replace=False) for _ in range(nlev)]) \
            if n else np.zeros((1, 1), dtype=np.int64)
        tok = np.zeros(n, dtype=np.int32)
        for u in range(n):
            for r, c in enumerate(kids[u]):
                tok[c] = table[lvl[c]][r % table.shape[1]]
        for u in range(n):
            if par[u] == -1:
                tok[u] = table[0][0]
        out.append(tok)
    return np.concatenate(out).astype(np.int32) if out else np.zeros(0, dtype=np.int32)


def make_verify_logits(cfg: Config, trees: list[np.ndarray], draft_tokens: np.ndarray, vocab: int = VOCAB,
                       match=MATCH, planted: float = 10.0) -> np.ndarray:
    """float32 [T][vocab] verify logits with one planted preferred token per row."""
    T = sum(len(t) for t in trees)
    logits = np.empty((T, vocab), dtype=np.float32)
    lo = 0
    for s, par in enumerate(trees):
        n = len(par)
        rng = _rng(cfg, _LOGITS, s)
        logits[lo:lo + n] = rng.standard_normal((n, vocab), dtype=np.float32)
        kids = _children_by_rank(par)
        u_draw = rng.random(n)
        for u in range(n):
            child_tok = [int(draft_tokens[lo + c]) for c in kids[u]]
            pick = -1
            acc = 0.0
            for r in range(len(child_tok)):
                acc += match[r] if r < len(match) else 0.0
                if u_draw[u] < acc:
                    pick = child_tok[r]
                    break
            if pick < 0:
                while True:
                    pick = int(rng.integers(vocab))
                    if pick not in child_tok or len(set(child_tok)) >= vocab:
                        break
            logits[lo + u, pick] = planted
        lo += n
    return logits


def make_draft_logits(cfg: Config, vocab: int = VOCAB, levels: int = DRAFT_LEVELS, width: int | None = None) -> np.ndarray:
    """float32 [B][levels][vocab]: the drafter's logits per drafted position."""
    width = cfg.tree[2] if width is None and cfg.tree[0] == "ddtree" else (width or 4)
    out = np.empty((cfg.num_seqs, levels, vocab), dtype=np.float32)
    for s in range(cfg.num_seqs):
        rng = _rng(cfg, _DLOGITS, s)
        out[s] = rng.standard_normal((levels, vocab), dtype=np.float32)
        for lvl in range(levels):
            w = min(width, vocab)
            toks = rng.choice(vocab, size=w, replace=False)
            out[s, lvl, toks] = (20.0 + rng.normal(0.0, 2.0, size=w)).astype(np.float32)
    return out


def make_root_tokens(cfg: Config, vocab: int = VOCAB) -> np.ndarray:
    """int32 [B]: each sequence's last committed token (the tree roots)."""
    return _rng(cfg, _ROOT, 0).integers(0, vocab, size=cfg.num_seqs).astype(np.int32)

"""Seeded per-node inputs, prefill tokens, accepted nodes and cache slots.

Value recipe (all configurations):
  q, k ~ N(0, 1), L2-normalized per (node, key head) in float64;
  v ~ N(0, 1);
  a = exp(-softplus(x)), b = sigmoid(y) with x, y ~ N(0, 1), in float64,
  stored as float32 (a is the decay gate, b the write strength);
  q/k/v are rounded float64 -> float32 (RNE) -> bfloat16 (RNE) for "bf16"
  configurations and kept as float32 for "f32".

Streams: numpy PCG64 seeded from ``SeedSequence(cfg.seed, spawn_key=...)``
with one key per (purpose, layer, sequence), so any slice of a workload can
be regenerated on its own.  bf16 values travel as their uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from .configs import Config
from .trees import chain_tree, ddtree_tree, random_tree

_TREE, _INPUT, _PREFILL, _MISC = 0, 1, 2, 3


def _rng(cfg: Config, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(cfg.seed, spawn_key=tuple(key))))


# ---------------------------------------------------------------- bf16 bits
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _unit_rows(g: np.ndarray) -> np.ndarray:
    return g / np.sqrt((g * g).sum(axis=-1, keepdims=True))


def _gates(rng: np.random.Generator, shape, a_low: float | None):
    x = rng.standard_normal(shape)
    y = rng.standard_normal(shape)
    if a_low is None:
        a = np.exp(-np.logaddexp(0.0, x))
    else:  # long-memory variant: a uniform in [a_low, 1)
        a = a_low + (1.0 - a_low) * rng.random(shape)
    b = 1.0 / (1.0 + np.exp(-y))
    return a.astype(np.float32), b.astype(np.float32)


# ---------------------------------------------------------------- structure
def make_trees(cfg: Config) -> list[np.ndarray]:
    """One parent array per sequence (shared by every layer of the step)."""
    trees = []
    for s in range(cfg.num_seqs):
        rng = _rng(cfg, _TREE, s)
        kind = cfg.tree[0]
        if kind == "chain":
            trees.append(chain_tree(cfg.tree[1]))
        elif kind == "random":
            trees.append(random_tree(rng, cfg.tree[1], cfg.tree[2]))
        elif kind == "ddtree":
            trees.append(ddtree_tree(rng, *cfg.tree[1:]))
        else:
            raise ValueError(kind)
    return trees


def cu_from_trees(trees: list[np.ndarray]) -> np.ndarray:
    cu = np.zeros(len(trees) + 1, dtype=np.int32)
    cu[1:] = np.cumsum([len(t) for t in trees])
    return cu


def make_accepts(cfg: Config, trees: list[np.ndarray]) -> np.ndarray:
    """Accepted end node per sequence (local id): a uniform leaf ("leaf"),
    node L-1 with L ~ U{1..n} ("chain_len"), or a uniform node ("node")."""
    rng = _rng(cfg, _MISC, 0)
    out = np.empty(len(trees), dtype=np.int32)
    for s, par in enumerate(trees):
        n = len(par)
        if cfg.accept == "leaf":
            has_child = np.zeros(n, dtype=bool)
            has_child[par[par >= 0]] = True
            leaves = np.flatnonzero(~has_child)
            out[s] = leaves[int(rng.integers(len(leaves)))]
        elif cfg.accept == "chain_len":
            out[s] = int(rng.integers(1, n + 1)) - 1
        elif cfg.accept == "node":
            out[s] = int(rng.integers(n))
        else:
            raise ValueError(cfg.accept)
    return out


def make_slots(cfg: Config) -> np.ndarray:
    if not cfg.slot_perm:
        return np.arange(cfg.num_seqs, dtype=np.int32)
    rng = _rng(cfg, _MISC, 1)
    return rng.permutation(cfg.num_slots)[: cfg.num_seqs].astype(np.int32)


# ---------------------------------------------------------------- values
def make_layer_inputs(cfg: Config, layer: int, trees: list[np.ndarray], a_low: float | None = None) -> dict:
    """q, k [T, H_k, D]; v [T, H_v, D] (bf16 bits or f32); a, b [T, H_v] f32."""
    hk, hv, d = cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim
    qs, ks, vs, as_, bs = [], [], [], [], []
    for s, par in enumerate(trees):
        n = len(par)
        rng = _rng(cfg, _INPUT, layer, s)
        qs.append(_unit_rows(rng.standard_normal((n, hk, d))))
        ks.append(_unit_rows(rng.standard_normal((n, hk, d))))
        vs.append(rng.standard_normal((n, hv, d)))
        a, b = _gates(rng, (n, hv), a_low)
        as_.append(a)
        bs.append(b)

    def cat(xs, shape_tail):
        return np.concatenate(xs, axis=0) if xs else np.zeros((0,) + shape_tail)

    return {
        "q": _store(cat(qs, (hk, d)), cfg.dtype),
        "k": _store(cat(ks, (hk, d)), cfg.dtype),
        "v": _store(cat(vs, (hv, d)), cfg.dtype),
        "a": cat(as_, (hv,)).astype(np.float32),
        "b": cat(bs, (hv,)).astype(np.float32),
    }


def make_prefill(cfg: Config, layer: int, seqs=None, a_low: float | None = None) -> dict:
    """Prefill tokens that build each sequence's committed state from zero:
    k [S, P, H_k, D], v [S, P, H_v, D] (config dtype), a, b [S, P, H_v] f32,
    for the sequences listed in ``seqs`` (default: all)."""
    hk, hv, d, p = cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim, cfg.prefill_steps
    seqs = range(cfg.num_seqs) if seqs is None else seqs
    ks, vs, as_, bs = [], [], [], []
    for s in seqs:
        rng = _rng(cfg, _PREFILL, layer, s)
        ks.append(_unit_rows(rng.standard_normal((p, hk, d))))
        vs.append(rng.standard_normal((p, hv, d)))
        a, b = _gates(rng, (p, hv), a_low)
        as_.append(a)
        bs.append(b)
    return {
        "k": _store(np.stack(ks), cfg.dtype),
        "v": _store(np.stack(vs), cfg.dtype),
        "a": np.stack(as_),
        "b": np.stack(bs),
    }

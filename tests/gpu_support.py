"""Shared helpers of the GPU tests: seeded workloads on the device, and the
oracle's expectations for them.  The oracle only ever sees host copies of the
same inputs; nothing the GPU computes flows into an expected value."""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import workloads as W

TOL = 2e-3  # max |x - r| / max |r| per (sequence, head) slice


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_deltanet_tree_amd as G
    G.load_library()  # raises if the HIP library was not built
    return G


def to_dev(x: np.ndarray, dtype_name: str | None = None) -> torch.Tensor:
    if x.dtype == np.uint16:  # bf16 bit patterns
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def slice_rel_err(x: np.ndarray, r: np.ndarray) -> float:
    """max over leading slices of max|x-r| / max|r| (x == 0 required where r == 0)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if not np.isfinite(x).all():
        return float("inf")
    num = np.abs(x - r).max(axis=-1)
    den = np.abs(r).max(axis=-1)
    worst = 0.0
    for n, d in zip(num.ravel(), den.ravel()):
        if d == 0:
            if n != 0:
                return float("inf")
        else:
            worst = max(worst, n / d)
    return worst


@functools.lru_cache(maxsize=8)
def host_case(name: str, layer: int = 0, a_low=None, extra_slots: int = 0):
    """Host-side inputs + oracle expectations for one configuration."""
    cfg = W.get_config(name)
    trees = W.make_trees(cfg)
    cu = W.cu_from_trees(trees)
    inp = W.make_layer_inputs(cfg, layer, trees, a_low=a_low)
    pre = W.make_prefill(cfg, layer, a_low=a_low)
    S0 = oracle.initial_states(pre, cfg.num_v_heads, cfg.head_dim)
    slots = W.make_slots(cfg)
    acc = W.make_accepts(cfg, trees)
    num_slots = cfg.num_slots + extra_slots
    # unused slots hold a sentinel pattern that no kernel may read into a result or overwrite
    rng = np.random.default_rng(99)
    cache = rng.standard_normal((num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim)).astype(np.float32)
    for s in range(cfg.num_seqs):
        cache[slots[s]] = S0[s]
    exp_out = oracle.verify_batch(trees, cu, inp, S0)
    exp_persist = oracle.persist_batch(trees, cu, inp, S0, acc)
    return dict(cfg=cfg, trees=trees, cu=cu, inp=inp, S0=S0, slots=slots, acc=acc, cache=cache,
                num_slots=num_slots, exp_out=exp_out, exp_persist=exp_persist)


def dims_for(G, case, total_nodes=None, max_nodes=None):
    cfg = case["cfg"]
    return G.make_dims(
        num_seqs=cfg.num_seqs, total_nodes=int(case["cu"][-1]) if total_nodes is None else total_nodes,
        max_nodes=cfg.max_nodes if max_nodes is None else max_nodes, num_k_heads=cfg.num_k_heads,
        num_v_heads=cfg.num_v_heads, head_dim=cfg.head_dim, num_slots=case["num_slots"],
        qkv_dtype=G.GDN_F32 if cfg.dtype == "f32" else G.GDN_BF16, max_depth=cfg.max_depth)


def device_case(G, case):
    d = {k: to_dev(v) for k, v in case["inp"].items()}
    d["parent"] = to_dev(np.concatenate(case["trees"]).astype(np.int32))
    d["cu"] = to_dev(case["cu"].astype(np.int32))
    d["slots"] = to_dev(case["slots"].astype(np.int32))
    d["acc"] = to_dev(case["acc"].astype(np.int32))
    d["cache"] = to_dev(case["cache"].copy())
    cfg = case["cfg"]
    d["out"] = torch.full((int(case["cu"][-1]), cfg.num_v_heads, cfg.head_dim), float("nan"),
                          dtype=torch.float32, device="cuda")
    d["dims"] = dims_for(G, case)
    d["ws"] = G.new_workspace(d["dims"])
    return d


def run_step(G, d, persist=True):
    """plan -> verify -> (persist) on the current stream."""
    G.gdn_tree_plan(d["dims"], d["parent"], d["cu"], d["slots"], d["ws"])
    G.gdn_tree_verify(d["dims"], d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], d["slots"], d["out"], d["ws"])
    if persist:
        G.gdn_tree_persist(d["dims"], d["k"], d["v"], d["a"], d["b"], d["acc"], d["cache"], d["slots"], d["ws"])
    torch.cuda.synchronize()

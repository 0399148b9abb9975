"""A seeded sweep over shapes the other GPU tests pin one at a time: batch size,
tree sizes on both sides of the 32- and 96-node kernel boundaries, head
groupings of 1-4 value heads per key head, head widths 16-128, bf16 and fp32
inputs, gate ranges, forests, node labelings out of topological order,
skipped sequences and slot permutations.  Every output and every persisted
state is checked against the oracle, and every other slot must stay untouched."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

CASES = 16


def _unit(rng, *shape):
    g = rng.standard_normal(shape)
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    d_, qkv = [(16, "f32"), (32, "f32"), (64, "bf16"), (128, "bf16"), (64, "f32"), (128, "bf16")][seed % 6]
    hk = int(rng.choice([1, 2, 4]))
    grp = int(rng.integers(1, 5))
    hv = hk * grp
    B = int(rng.integers(1, 12))
    size_band = [(1, 8), (20, 33), (30, 65), (60, 97), (90, 130)][seed % 5]
    sizes = rng.integers(size_band[0], size_band[1] + 1, size=B)
    sizes[rng.random(B) < 0.1] = 0  # an empty sequence now and then
    trees = []
    for n in sizes:
        n = int(n)
        if n == 0:
            trees.append(np.zeros(0, np.int32))
            continue
        par = W.random_tree(rng, n, int(rng.integers(2, 17)))
        if rng.random() < 0.3 and n > 2:  # a second root: a forest
            par[int(rng.integers(1, n))] = -1
        if rng.random() < 0.5:  # relabel out of topological order
            par = W.relabel(par, rng.permutation(n))
        trees.append(par.astype(np.int32))
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum([len(t) for t in trees])
    T = int(cu[-1])
    lo_a = float(rng.choice([0.05, 0.5, 0.9]))
    inp = {"q": _unit(rng, T, hk, d_), "k": _unit(rng, T, hk, d_), "v": rng.standard_normal((T, hv, d_)),
           "a": rng.uniform(lo_a, 1.0, (T, hv)), "b": rng.uniform(0.0, 1.0, (T, hv))}
    inp = {k: v.astype(np.float32) for k, v in inp.items()}
    if qkv == "bf16":
        for key in ("q", "k", "v"):
            inp[key] = W.f32_to_bf16_bits(inp[key])
    n_slots = B + int(rng.integers(0, 4))
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    cache = (0.3 * rng.standard_normal((n_slots, hv, d_, d_))).astype(np.float32)
    acc = np.array([int(rng.integers(-1, len(t))) if len(t) else -1 for t in trees], np.int32)
    return dict(d=d_, qkv=qkv, hk=hk, hv=hv, B=B, trees=trees, cu=cu, T=T, inp=inp, slots=slots, cache=cache,
                acc=acc, max_nodes=max([len(t) for t in trees] + [1]))


@pytest.mark.parametrize("seed", range(CASES))
def test_sweep(seed, monkeypatch):
    G = require_gpu()
    c = _case(seed)
    # odd cases fix the verify's head grouping to shared workgroups (the automatic
    # choice at these batch sizes is one value head per workgroup)
    heads = "shared" if seed % 2 else "auto"
    if heads == "auto":
        monkeypatch.delenv("GDN_VERIFY_HEADS", raising=False)
    else:
        monkeypatch.setenv("GDN_VERIFY_HEADS", heads)
    print("sweep case", seed, "d", c["d"], c["qkv"], "heads", c["hk"], c["hv"], "B", c["B"],
          "nodes", [len(t) for t in c["trees"]], "grouping", heads, flush=True)
    T, hv, d_ = c["T"], c["hv"], c["d"]
    dims = G.make_dims(c["B"], T, c["max_nodes"], c["hk"], hv, d_, len(c["cache"]),
                       G.GDN_BF16 if c["qkv"] == "bf16" else G.GDN_F32)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in c["inp"].items()}
    cache_d = to_dev(c["cache"])
    slots_d = to_dev(c["slots"])
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    parent = np.concatenate(c["trees"]) if T else np.zeros(0, np.int32)
    G.gdn_tree_plan(dims, to_dev(parent.astype(np.int32)), to_dev(c["cu"]), slots_d, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, slots_d, out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(c["acc"]), cache_d, slots_d, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    got = out.cpu().numpy()[:T]
    after = cache_d.cpu().numpy()
    S0 = c["cache"][c["slots"]]
    ref = oracle.verify_batch(c["trees"], c["cu"], c["inp"], S0)
    persisted = oracle.persist_batch(c["trees"], c["cu"], c["inp"], S0, c["acc"])
    for s in range(c["B"]):
        lo, hi = int(c["cu"][s]), int(c["cu"][s + 1])
        if hi > lo:
            assert slice_rel_err(got[lo:hi].transpose(1, 0, 2).reshape(hv, -1),
                                 ref[lo:hi].transpose(1, 0, 2).reshape(hv, -1)) <= TOL, ("out", s)
        st, _ = persisted[s]
        slot = int(c["slots"][s])
        if st is None:
            assert np.array_equal(after[slot].view(np.uint32), c["cache"][slot].view(np.uint32)), ("skipped", s)
        else:
            assert slice_rel_err(after[slot].reshape(hv, -1), st.reshape(hv, -1)) <= TOL, ("state", s)
    spare = np.setdiff1d(np.arange(len(c["cache"])), c["slots"])
    assert np.array_equal(after[spare].view(np.uint32), c["cache"][spare].view(np.uint32))

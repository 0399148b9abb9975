"""Trees of 97-256 nodes on the matrix cores (the coefficient + verify pair).

Each case is a ragged batch: one large tree (random attachment, a DDTree grown
to the budget with depth 16, a forest, or a relabelled tree whose ancestors sit
in later node blocks than their descendants), a small tree and an empty
sequence, against the oracle to the per-slice tolerance, with persist and a
spare cache slot that must stay untouched.  A key-head group too wide for the
pair's LDS takes the recurrent walk and is checked the same way."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _inputs(rng, T, hk, hv, d):
    q = rng.standard_normal((T, hk, d))
    k = rng.standard_normal((T, hk, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return {"q": W.f32_to_bf16_bits(q.astype(np.float32)), "k": W.f32_to_bf16_bits(k.astype(np.float32)),
            "v": W.f32_to_bf16_bits(rng.standard_normal((T, hv, d)).astype(np.float32)),
            "a": rng.uniform(0.3, 1.0, (T, hv)).astype(np.float32),
            "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}


def _large_tree(rng, shape):
    if shape == "random97":
        return W.random_tree(rng, 97, 16)
    if shape == "ddtree256":
        par = W.ddtree_tree(rng, 255, 16, 16)
        assert len(par) == 256 and W.tree_depths(par).max() == 16
        return par
    if shape == "forest130":  # three roots: 60 + 50 + 20 nodes
        parts, off = [], 0
        for n in (60, 50, 20):
            p = W.random_tree(rng, n, 16)
            parts.append(np.where(p >= 0, p + off, -1))
            off += n
        return np.concatenate(parts).astype(np.int32)
    if shape == "relabel200":
        par = W.ddtree_tree(rng, 199, 8, 16)
        return W.relabel(par, rng.permutation(len(par)))
    raise ValueError(shape)


def _run_case(G, rng, big, hk, hv, d_):
    trees = [big, W.random_tree(rng, 5, 4), np.zeros(0, np.int32)]
    B = len(trees)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    nmax = max(len(t) for t in trees)
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.array([2, 0, 1], np.int32)
    cache = np.full((B + 1, hv, d_, d_), 5.0, np.float32)
    for s in range(B):
        cache[slots[s]] = S0[s]
    acc = np.array([int(np.argmax(W.tree_depths(big))), 3, -1], np.int32)
    dims = G.make_dims(B, T, nmax, hk, hv, d_, B + 1, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    cache_d = to_dev(cache.copy())
    slots_d = to_dev(slots)
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)), slots_d, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, slots_d, out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(acc), cache_d, slots_d, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    got = out.cpu().numpy()
    exp = oracle.verify_batch(trees, cu, inp, S0)
    for s in range(B):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if hi > lo:
            x = got[lo:hi].transpose(1, 0, 2).reshape(hv, -1)
            r = exp[lo:hi].transpose(1, 0, 2).reshape(hv, -1)
            assert slice_rel_err(x, r) <= TOL, s
    res = oracle.persist_batch(trees, cu, inp, S0, acc)
    after = cache_d.cpu().numpy()
    for s in range(B):
        st, _ = res[s]
        if st is None:
            assert np.array_equal(after[slots[s]].view(np.uint32), cache[slots[s]].view(np.uint32))
        else:
            assert slice_rel_err(after[slots[s]].reshape(hv, -1), st.reshape(hv, -1)) <= TOL, s
    assert np.array_equal(after[B].view(np.uint32), cache[B].view(np.uint32))


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("shape", ["random97", "forest130", "relabel200", "ddtree256"])
def test_large_tree_on_matrix_cores(d_, shape, monkeypatch):
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    rng = np.random.default_rng(4000 + d_ + len(shape))
    big = _large_tree(rng, shape)
    print("large tree %s d=%d" % (shape, d_), flush=True)
    _run_case(G, rng, big, 2, 6, d_)


@pytest.mark.parametrize("heads_per_key", [1, 5])
def test_large_tree_head_groups(heads_per_key, monkeypatch):
    """One and five value heads per key head: the coefficient kernel's passes over
    the group's heads at 256 nodes."""
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    rng = np.random.default_rng(4100 + heads_per_key)
    big = W.ddtree_tree(rng, 255, 16, 16)
    print("large tree head groups %d" % heads_per_key, flush=True)
    _run_case(G, rng, big, 2, 2 * heads_per_key, 128)


def test_wide_key_head_group_falls_back():
    """48 value heads on one key head at 256 nodes: the coefficient tables would not
    fit one compute unit's LDS, so the recurrent walk verifies the tree."""
    G = require_gpu()
    rng = np.random.default_rng(4200)
    big = W.random_tree(rng, 256, 16)
    print("wide key-head group", flush=True)
    _run_case(G, rng, big, 1, 48, 64)

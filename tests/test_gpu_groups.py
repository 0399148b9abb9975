"""Parity across value-heads-per-key-head ratios (1..5) and head sizes 64/128.

Trees of at most 32 nodes run the group kernel and trees of 33-96 nodes the
node-block kernel; chains of at most 16 nodes run the group kernel through
gdn_chain_verify.  Under GDN_VERIFY_HEADS=shared a workgroup takes all value
heads of its key head (1..4; the coefficient + verify pair beyond); these
batches are small, so the automatic choice gives each value head its own
workgroup (any ratio).  Both are run.  Each case is a ragged batch with an
empty sequence and a forest, checked against the oracle to the per-slice
tolerance."""
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


def _check_out(got, exp, cu, hv):
    for s in range(len(cu) - 1):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if hi > lo:
            x = got[lo:hi].transpose(1, 0, 2).reshape(hv, -1)
            r = exp[lo:hi].transpose(1, 0, 2).reshape(hv, -1)
            assert slice_rel_err(x, r) <= TOL, s


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("grp", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("big", [False, True])
@pytest.mark.parametrize("heads", ["auto", "shared"])
def test_tree_head_groups(d_, grp, big, heads, monkeypatch):
    G = require_gpu()
    if heads == "auto":  # this batch is small: one value head per verify workgroup
        monkeypatch.delenv("GDN_VERIFY_HEADS", raising=False)
    else:
        monkeypatch.setenv("GDN_VERIFY_HEADS", heads)
    rng = np.random.default_rng(1000 * grp + d_ + (7 if big else 0))
    hk = 2
    hv = hk * grp
    nmax = 40 if big else 32
    trees = [W.random_tree(rng, 11, 6), np.zeros(0, np.int32), np.array([-1, 0, -1, 2, 2, 1], np.int32),
             W.random_tree(rng, nmax, 16), W.chain_tree(16)]
    B = len(trees)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.array([2, 0, 4, 1, 3], np.int32)
    cache = np.full((B + 1, hv, d_, d_), 5.0, np.float32)
    for s in range(B):
        cache[slots[s]] = S0[s]
    acc = np.array([10, -1, 5, nmax - 1, 15], np.int32)
    dims = G.make_dims(B, T, nmax, hk, hv, d_, B + 1, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    cache_d = to_dev(cache.copy())
    slots_d = to_dev(slots)
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    print("tree head groups d=%d grp=%d nmax=%d heads=%s" % (d_, grp, nmax, heads), flush=True)
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)), slots_d, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, slots_d, out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(acc), cache_d, slots_d, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    _check_out(out.cpu().numpy(), oracle.verify_batch(trees, cu, inp, S0), cu, hv)
    res = oracle.persist_batch(trees, cu, inp, S0, acc)
    after = cache_d.cpu().numpy()
    for s in range(B):
        st, _ = res[s]
        if st is None:
            assert np.array_equal(after[slots[s]].view(np.uint32), cache[slots[s]].view(np.uint32))
        else:
            assert slice_rel_err(after[slots[s]].reshape(hv, -1), st.reshape(hv, -1)) <= TOL
    assert np.array_equal(after[B].view(np.uint32), cache[B].view(np.uint32))


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("grp", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("heads", ["auto", "shared"])
def test_chain_head_groups(d_, grp, heads, monkeypatch):
    G = require_gpu()
    if heads == "auto":
        monkeypatch.delenv("GDN_VERIFY_HEADS", raising=False)
    else:
        monkeypatch.setenv("GDN_VERIFY_HEADS", heads)
    rng = np.random.default_rng(2000 * grp + d_)
    hk = 2
    hv = hk * grp
    lens = [16, 0, 1, 9, 16]
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.array([3, 1, 0, 4, 2], np.int32)
    cache = np.zeros((B, hv, d_, d_), np.float32)
    for s in range(B):
        cache[slots[s]] = S0[s]
    final_len = np.array([16, 0, 1, 4, 0], np.int32)
    dims = G.make_dims(B, T, 16, hk, hv, d_, B, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    fin = torch.full((B, hv, d_, d_), float("nan"), device="cuda")
    print("chain head groups d=%d grp=%d heads=%s" % (d_, grp, heads), flush=True)
    G.gdn_chain_verify(dims, to_dev(cu.astype(np.int32)), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"],
                       to_dev(cache), to_dev(slots), out, to_dev(final_len), fin, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    got = out.cpu().numpy()
    fin_h = fin.cpu().numpy()
    for s in range(B):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = slice(lo, hi)
        o, _ = oracle.chain(inp["k"][sl], inp["v"][sl], inp["a"][sl], inp["b"][sl], S0[s], q=inp["q"][sl])
        if hi > lo:
            assert slice_rel_err(got[sl].transpose(1, 0, 2).reshape(hv, -1),
                                 o.transpose(1, 0, 2).reshape(hv, -1)) <= TOL, s
        m = int(final_len[s])
        _, st = oracle.chain(inp["k"][lo:lo + m], inp["v"][lo:lo + m], inp["a"][lo:lo + m], inp["b"][lo:lo + m], S0[s])
        if m == 0:
            assert np.array_equal(fin_h[s], S0[s])
        else:
            assert slice_rel_err(fin_h[s].reshape(hv, -1), st.reshape(hv, -1)) <= TOL, s


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("n_nodes", [40, 65, 96])
def test_relabelled_multi_block_trees(d_, n_nodes):
    """Trees of 33-96 nodes with shuffled labels, so ancestors sit in later node
    blocks than their descendants; outputs checked against the oracle."""
    G = require_gpu()
    rng = np.random.default_rng(3000 + n_nodes + d_)
    hk, hv = 2, 6
    trees = []
    for _ in range(3):
        par = W.random_tree(rng, n_nodes, 16)
        trees.append(W.relabel(par, rng.permutation(n_nodes)))
    B = len(trees)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.array([1, 2, 0], np.int32)
    cache = np.zeros((B, hv, d_, d_), np.float32)
    for s in range(B):
        cache[slots[s]] = S0[s]
    dims = G.make_dims(B, T, n_nodes, hk, hv, d_, B, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    print("relabelled multi-block d=%d n=%d" % (d_, n_nodes), flush=True)
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)),
                    to_dev(slots), ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], to_dev(cache), to_dev(slots), out, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    _check_out(out.cpu().numpy(), oracle.verify_batch(trees, cu, inp, S0), cu, hv)

"""fp32 q/k/v on the matrix cores (head sizes 64 and 128).

Keys and queries enter the products split into bf16 hi + lo and values stay
fp32, so outputs and persisted states keep about 16 significant bits: every
case is held to 1e-4 per (sequence, head) slice, twenty times tighter than the
parity bar and well below what rounding the inputs to bf16 would give (about
2e-3).  Trees of up to 32 nodes run the group kernel (one and all value heads
per workgroup), larger ones the coefficient + verify pair; chains run the group
kernel and the replay; persist runs the replay."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4


def _inputs(rng, T, hk, hv, d):
    q = rng.standard_normal((T, hk, d))
    k = rng.standard_normal((T, hk, d))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return {"q": q.astype(np.float32), "k": k.astype(np.float32),
            "v": rng.standard_normal((T, hv, d)).astype(np.float32),
            "a": rng.uniform(0.3, 1.0, (T, hv)).astype(np.float32),
            "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}


def _trees(rng, kind):
    if kind == "small":  # the group kernel: <= 32 nodes, a forest, an empty sequence
        return [W.random_tree(rng, 11, 6), np.zeros(0, np.int32), np.array([-1, 0, -1, 2, 2, 1], np.int32),
                W.ddtree_tree(rng, 31, 4, 16), W.chain_tree(16)]
    if kind == "blocks":  # 33-96 nodes: the pair for fp32 inputs
        return [W.ddtree_tree(rng, 64, 8, 16), W.random_tree(rng, 40, 16), np.zeros(0, np.int32)]
    if kind == "large":  # 97-256 nodes
        return [W.relabel(W.ddtree_tree(rng, 199, 8, 16), rng.permutation(200)), W.random_tree(rng, 7, 4)]
    raise ValueError(kind)


def _accepts(trees):
    return np.array([int(np.argmax(W.tree_depths(t))) if len(t) else -1 for t in trees], np.int32)


@pytest.mark.parametrize("d_", [64, 128])
@pytest.mark.parametrize("kind,heads", [("small", "auto"), ("small", "shared"), ("blocks", "auto"),
                                        ("large", "auto")])
def test_f32_tree_verify_and_persist(d_, kind, heads, monkeypatch):
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    if heads == "auto":
        monkeypatch.delenv("GDN_VERIFY_HEADS", raising=False)
    else:
        monkeypatch.setenv("GDN_VERIFY_HEADS", heads)
    rng = np.random.default_rng(5000 + d_ + len(kind) + len(heads))
    trees = _trees(rng, kind)
    hk, hv = 2, 6
    B = len(trees)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    nmax = max(len(t) for t in trees)
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = rng.permutation(B).astype(np.int32)
    cache = np.full((B + 1, hv, d_, d_), 5.0, np.float32)
    for s in range(B):
        cache[slots[s]] = S0[s]
    acc = _accepts(trees)
    dims = G.make_dims(B, T, nmax, hk, hv, d_, B + 1, G.GDN_F32)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    cache_d = to_dev(cache.copy())
    slots_d = to_dev(slots)
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    print("f32 inputs %s d=%d heads=%s" % (kind, d_, heads), flush=True)
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
            assert slice_rel_err(x, r) <= F32_TOL, (s, slice_rel_err(x, r))
    res = oracle.persist_batch(trees, cu, inp, S0, acc)
    after = cache_d.cpu().numpy()
    for s in range(B):
        st, _ = res[s]
        if st is None:
            assert np.array_equal(after[slots[s]].view(np.uint32), cache[slots[s]].view(np.uint32))
        else:
            assert slice_rel_err(after[slots[s]].reshape(hv, -1), st.reshape(hv, -1)) <= F32_TOL, s
    assert np.array_equal(after[B].view(np.uint32), cache[B].view(np.uint32))


@pytest.mark.parametrize("d_", [64, 128])
def test_f32_chain_and_final_states(d_, monkeypatch):
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    rng = np.random.default_rng(5100 + d_)
    hk, hv = 2, 6
    lens = [16, 0, 1, 9, 16]
    B = len(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T = int(cu[-1])
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.arange(B, dtype=np.int32)
    final_len = np.array([16, 0, 1, 4, 9], np.int32)
    dims = G.make_dims(B, T, 16, hk, hv, d_, B, G.GDN_F32)
    ws = G.new_workspace(dims)
    dev = {k_: to_dev(v_) for k_, v_ in inp.items()}
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    fin = torch.full((B, hv, d_, d_), float("nan"), device="cuda")
    print("f32 chains d=%d" % d_, flush=True)
    G.gdn_chain_verify(dims, to_dev(cu), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], to_dev(S0),
                       to_dev(slots), out, to_dev(final_len), fin, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    got, fin_h = out.cpu().numpy(), fin.cpu().numpy()
    for s in range(B):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = slice(lo, hi)
        o, _ = oracle.chain(inp["k"][sl], inp["v"][sl], inp["a"][sl], inp["b"][sl], S0[s], q=inp["q"][sl])
        if hi > lo:
            assert slice_rel_err(got[sl].transpose(1, 0, 2).reshape(hv, -1),
                                 o.transpose(1, 0, 2).reshape(hv, -1)) <= F32_TOL, s
        m = int(final_len[s])
        _, st = oracle.chain(inp["k"][lo:lo + m], inp["v"][lo:lo + m], inp["a"][lo:lo + m], inp["b"][lo:lo + m],
                             S0[s])
        if m == 0:
            assert np.array_equal(fin_h[s], S0[s])
        else:
            assert slice_rel_err(fin_h[s].reshape(hv, -1), st.reshape(hv, -1)) <= F32_TOL, s


def test_f32_split_beats_bf16_rounding(monkeypatch):
    """The same fp32 inputs rounded to bf16 first move the outputs by far more than
    the split's error: the kernels do use the inputs' low bits."""
    G = require_gpu()
    monkeypatch.delenv("GDN_KERNEL_PATH", raising=False)
    rng = np.random.default_rng(5200)
    trees = [W.ddtree_tree(rng, 22, 4, 16) for _ in range(4)]
    hk, hv, d_ = 2, 6, 128
    B = len(trees)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    inp = _inputs(rng, T, hk, hv, d_)
    S0 = (0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32)
    slots = np.arange(B, dtype=np.int32)
    dims = G.make_dims(B, T, 23, hk, hv, d_, B, G.GDN_F32)
    ws = G.new_workspace(dims)
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)),
                    to_dev(slots), ws)
    errs = []
    for rounded in (False, True):
        x = {k_: (W.bf16_bits_to_f32(W.f32_to_bf16_bits(v_)) if rounded and k_ in "qkv" else v_)
             for k_, v_ in inp.items()}
        dev = {k_: to_dev(np.ascontiguousarray(v_, np.float32)) for k_, v_ in x.items()}
        out = torch.full((T, hv, d_), float("nan"), device="cuda")
        G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], to_dev(S0), to_dev(slots), out, ws)
        torch.cuda.synchronize()
        exp = oracle.verify_batch(trees, cu, inp, S0)
        got = out.cpu().numpy()
        errs.append(max(slice_rel_err(got[cu[s]:cu[s + 1]].transpose(1, 0, 2).reshape(hv, -1),
                                      exp[cu[s]:cu[s + 1]].transpose(1, 0, 2).reshape(hv, -1)) for s in range(B)))
    assert errs[0] <= F32_TOL and errs[1] > 10 * errs[0], errs

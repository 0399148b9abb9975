"""Error paths on the GPU: malformed trees, bad slots and accepted nodes are
rejected per sequence, with the verdict the CPU validator predicts, NaN
outputs, and an untouched cache slot; healthy sequences in the same call are
unaffected.  Host-side argument errors return before any launch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import plan as P
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu

HK, HV = 2, 4
# (head dim, q/k/v storage): D=16 fp32 runs the recurrent kernels, D=64 bf16 the MFMA kernels
PATHS = {"recurrent": (16, "f32"), "mfma": (64, "bf16")}


def _base(rng, n_each=(7, 9, 6, 8)):
    trees = [W.random_tree(rng, n, 6) for n in n_each]
    return trees


def _inputs(rng, T, D, dt):
    q = rng.standard_normal((T, HK, D))
    k = rng.standard_normal((T, HK, D))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, HV, D))
    cast = (lambda x: x.astype(np.float32)) if dt == "f32" else (lambda x: W.f32_to_bf16_bits(x.astype(np.float32)))
    return {"q": cast(q), "k": cast(k), "v": cast(v),
            "a": rng.uniform(0.3, 1.0, (T, HV)).astype(np.float32),
            "b": rng.uniform(0.0, 1.0, (T, HV)).astype(np.float32)}


CASES = {
    "bad_parent_range": lambda t, s, c: (t[1].__setitem__(3, 42), s, c),
    "self_parent": lambda t, s, c: (t[1].__setitem__(2, 2), s, c),
    "cycle": lambda t, s, c: (t[1].__setitem__(1, 4) or t[1].__setitem__(4, 1) or t[1].__setitem__(0, -1), s, c),
    "too_deep": None,  # built below
    "bad_slot": lambda t, s, c: (None, s.__setitem__(1, 17), c),
    "dup_slot": lambda t, s, c: (None, s.__setitem__(1, int(s[3])), c),
    "bad_range": None,  # built below
}


def _make(name, rng):
    trees = _base(rng)
    slots = np.array([3, 1, 0, 2], np.int32)
    cu = W.cu_from_trees(trees)
    max_depth = 6
    max_nodes = 16
    if name == "too_deep":
        trees[1] = W.chain_tree(9)  # depth 9 > max_depth 6
        cu = W.cu_from_trees(trees)
    elif name == "bad_range":
        max_nodes = 8  # sequence 1 has 9 nodes
    else:
        trees = [t.copy() for t in trees]
        CASES[name](trees, slots, cu)
        cu = W.cu_from_trees(trees)
    return trees, slots, cu, max_depth, max_nodes


@pytest.mark.parametrize("path", sorted(PATHS))
@pytest.mark.parametrize("name", ["bad_parent_range", "self_parent", "cycle", "too_deep", "bad_slot",
                                  "dup_slot", "bad_range"])
def test_rejected_sequence(name, path):
    G = require_gpu()
    D, dt = PATHS[path]
    rng = np.random.default_rng(sum(map(ord, name)))
    trees, slots, cu, max_depth, max_nodes = _make(name, rng)
    parent = np.concatenate(trees).astype(np.int32)
    T = len(parent)
    num_slots = 4
    expect = P.validate(parent, cu, slots, num_slots, max_nodes, max_depth)
    assert (expect != 0).any()
    inp = _inputs(rng, T, D, dt)
    cache = rng.standard_normal((num_slots, HV, D, D)).astype(np.float32)
    dims = G.make_dims(4, T, max_nodes, HK, HV, D, num_slots, G.GDN_F32 if dt == "f32" else G.GDN_BF16,
                       max_depth=max_depth)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in inp.items()}
    cache_d = to_dev(cache.copy())
    out = torch.zeros((T, HV, D), device="cuda")
    acc = np.array([0, 0, 0, 0], np.int32)
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu.astype(np.int32)), to_dev(slots), ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, to_dev(slots), out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(acc), cache_d, to_dev(slots), ws)
    rc, bad, code = G.gdn_tree_status(ws)
    md = G.read_metadata(dims, ws)
    got = md["seq_status"].cpu().numpy()
    assert np.array_equal(got, expect), (got, expect)
    first = int(np.flatnonzero(expect)[0])
    assert (rc, bad, code) == (-6, first, int(expect[first]))
    o = out.cpu().numpy()
    after = cache_d.cpu().numpy()
    for s in range(4):
        lo, hi = int(cu[s]), int(cu[s + 1])
        ok_range = 0 <= lo <= hi <= T
        if expect[s] != 0:
            if ok_range and hi > lo:
                assert np.isnan(o[lo:hi]).all()
            if 0 <= slots[s] < num_slots and not any(
                    expect[t] == 0 and slots[t] == slots[s] for t in range(4)):
                assert np.array_equal(after[slots[s]].view(np.uint32), cache[slots[s]].view(np.uint32))
        else:
            exp = oracle.tree(trees[s], inp["q"][lo:hi], inp["k"][lo:hi], inp["v"][lo:hi],
                              inp["a"][lo:hi], inp["b"][lo:hi], cache[slots[s]])
            x = o[lo:hi].transpose(1, 0, 2).reshape(HV, -1)
            assert slice_rel_err(x, exp.transpose(1, 0, 2).reshape(HV, -1)) <= TOL
            st, _ = oracle.accept_state(trees[s], 0, inp["k"][lo:hi], inp["v"][lo:hi], inp["a"][lo:hi],
                                        inp["b"][lo:hi], cache[slots[s]])
            assert slice_rel_err(after[slots[s]].reshape(HV, -1), st.reshape(HV, -1)) <= TOL


@pytest.mark.parametrize("path", sorted(PATHS))
def test_bad_accepted_node(path):
    G = require_gpu()
    D, dt = PATHS[path]
    rng = np.random.default_rng(4)
    trees = _base(rng)
    parent = np.concatenate(trees).astype(np.int32)
    cu = W.cu_from_trees(trees)
    T = len(parent)
    slots = np.array([0, 1, 2, 3], np.int32)
    inp = _inputs(rng, T, D, dt)
    cache = rng.standard_normal((4, HV, D, D)).astype(np.float32)
    dims = G.make_dims(4, T, 16, HK, HV, D, 4, G.GDN_F32 if dt == "f32" else G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in inp.items()}
    cache_d = to_dev(cache.copy())
    acc = np.array([1, len(trees[1]), -1, -2], np.int32)  # seq 1: one past the end; seq 3: below -1
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu.astype(np.int32)), to_dev(slots), ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(acc), cache_d, to_dev(slots), ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert (rc, bad, code) == (-6, 1, P.SEQ_BAD_ACCEPT)
    md = G.read_metadata(dims, ws)
    assert list(md["seq_status"].cpu().numpy()) == [0, P.SEQ_BAD_ACCEPT, 0, P.SEQ_BAD_ACCEPT]
    after = cache_d.cpu().numpy()
    for s in (1, 2, 3):
        assert np.array_equal(after[s].view(np.uint32), cache[s].view(np.uint32))
    assert md["path_len"].cpu().numpy()[2] == 0
    assert not np.array_equal(after[0], cache[0])


def test_host_side_errors():
    G = require_gpu()
    dims = G.make_dims(1, 4, 8, 1, 1, 16, 1, G.GDN_F32)
    ws = G.new_workspace(dims)
    par = to_dev(np.array([-1, 0, 0, 1], np.int32))
    cu = to_dev(np.array([0, 4], np.int32))
    sl = to_dev(np.array([0], np.int32))
    with pytest.raises(G.GdnError) as e:
        G.gdn_tree_plan(dims, par, cu, sl, ws[:16])
    assert e.value.code == -4
    bad = G.make_dims(1, 4, 8, 1, 1, 48, 1, G.GDN_F32)
    with pytest.raises(G.GdnError) as e:
        G.gdn_tree_plan(bad, par, cu, sl, ws)
    assert e.value.code == -3
    bad = G.make_dims(1, 4, 8, 2, 3, 16, 1, G.GDN_F32)  # 3 value heads over 2 key heads
    with pytest.raises(G.GdnError) as e:
        G.gdn_tree_plan(bad, par, cu, sl, ws)
    assert e.value.code == -2
    bad = G.make_dims(1, 4, 300, 1, 1, 16, 1, G.GDN_F32)  # more than GDN_MAX_NODES
    with pytest.raises(G.GdnError) as e:
        G.gdn_tree_plan(bad, par, cu, sl, ws)
    assert e.value.code == -2
    with pytest.raises(TypeError):
        G.gdn_tree_plan(dims, par.float(), cu, sl, ws)
    fresh = torch.zeros_like(ws)
    rc, _, _ = G.gdn_tree_status(fresh)
    assert rc == -4  # never planned


def _misuse_case(G, D, dt, rng):
    trees = _base(rng)
    parent = np.concatenate(trees).astype(np.int32)
    cu = W.cu_from_trees(trees).astype(np.int32)
    T = len(parent)
    slots = np.array([2, 0, 3, 1], np.int32)
    inp = _inputs(rng, T, D, dt)
    cache = rng.standard_normal((4, HV, D, D)).astype(np.float32)
    qkv = G.GDN_F32 if dt == "f32" else G.GDN_BF16
    return parent, cu, T, slots, inp, cache, qkv


def _tree_calls_write_nothing(G, dims, ws, T, D, dev, cache, cache_d, slots, accept_vocab=37):
    """verify, persist and accept on a workspace whose plan does not match `dims`:
    outputs keep their sentinel, no slot changes, acceptance reports nothing, and
    gdn_tree_status names the workspace."""
    sentinel = 123.25
    out = torch.full((T, HV, D), sentinel, device="cuda")
    acc = to_dev(np.zeros(4, np.int32))
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, to_dev(slots), out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], acc, cache_d, to_dev(slots), ws)
    logits = torch.zeros((T, accept_vocab), device="cuda")
    tok = torch.zeros(T, dtype=torch.int32, device="cuda")
    a_out, l_out, n_out = (torch.full((4,), 77, dtype=torch.int32, device="cuda") for _ in range(3))
    G.gdn_tree_accept(dims, logits, tok, a_out, l_out, n_out, ws)
    rc, _, _ = G.gdn_tree_status(ws)
    assert rc == -4
    assert (out.cpu().numpy() == sentinel).all()
    assert np.array_equal(cache_d.cpu().numpy().view(np.uint32), cache.view(np.uint32))
    assert a_out.cpu().tolist() == [-1] * 4 and l_out.cpu().tolist() == [0] * 4
    assert n_out.cpu().tolist() == [-1] * 4


@pytest.mark.parametrize("path", sorted(PATHS))
def test_plan_for_other_dims_is_rejected(path):
    """A plan made with a larger max_nodes (or another max_depth) than the calls
    that read it: verify, persist and accept write nothing, and the status call
    reports the workspace; the same calls with the plan's own dims work."""
    G = require_gpu()
    D, dt = PATHS[path]
    rng = np.random.default_rng(31)
    parent, cu, T, slots, inp, cache, qkv = _misuse_case(G, D, dt, rng)
    dev = {k: to_dev(v) for k, v in inp.items()}
    for plan_nodes, plan_depth, call_nodes, call_depth in ((64, 16, 16, 16), (16, 12, 16, 16)):
        plan_dims = G.make_dims(4, T, plan_nodes, HK, HV, D, 4, qkv, max_depth=plan_depth)
        dims = G.make_dims(4, T, call_nodes, HK, HV, D, 4, qkv, max_depth=call_depth)
        ws = G.new_workspace(dims)
        cache_d = to_dev(cache.copy())
        G.gdn_tree_plan(plan_dims, to_dev(parent), to_dev(cu), to_dev(slots), ws)
        _tree_calls_write_nothing(G, dims, ws, T, D, dev, cache, cache_d, slots)
        # planned again for the calls' dims, the same workspace works
        G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu), to_dev(slots), ws)
        out = torch.full((T, HV, D), float("nan"), device="cuda")
        G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, to_dev(slots), out, ws)
        assert G.gdn_tree_status(ws)[0] == 0
        assert np.isfinite(out.cpu().numpy()).all()


@pytest.mark.parametrize("path", sorted(PATHS))
def test_chain_workspace_is_not_a_plan(path):
    """gdn_chain_verify marks its workspace as a chain workspace: the status call
    reads its verdicts, and the tree calls refuse it (it holds no paths or
    preorder) until it is planned again."""
    G = require_gpu()
    D, dt = PATHS[path]
    rng = np.random.default_rng(32)
    parent, cu, T, slots, inp, cache, qkv = _misuse_case(G, D, dt, rng)
    dev = {k: to_dev(v) for k, v in inp.items()}
    dims = G.make_dims(4, T, 16, HK, HV, D, 4, qkv)
    ws = G.new_workspace(dims)
    cache_d = to_dev(cache.copy())
    # a real plan first, so the chain call overwrites a valid header
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu), to_dev(slots), ws)
    cout = torch.full((T, HV, D), float("nan"), device="cuda")
    G.gdn_chain_verify(dims, to_dev(cu), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, to_dev(slots),
                       cout, ws=ws)
    assert G.gdn_tree_status(ws)[0] == 0
    assert np.isfinite(cout.cpu().numpy()).all()
    _tree_calls_write_nothing(G, dims, ws, T, D, dev, cache, cache_d, slots)

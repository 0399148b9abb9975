"""GPU parity at the edges: long chains (chunked), the largest tree a call
accepts, and the stress workload at full size over two layer calls."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _unit(rng, *shape):
    g = rng.standard_normal(shape)
    return g / np.linalg.norm(g, axis=-1, keepdims=True)


def _bf(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("d_", [32, 128])
def test_long_chain_outputs_and_final_states(d_):
    """Chains longer than one 16-node chunk, with final states taken at chunk
    boundaries and inside chunks."""
    G = require_gpu()
    rng = np.random.default_rng(21)
    hk, hv = 2, 4
    lens = [64, 17, 5, 40]
    fl = np.array([64, 16, 0, 33], np.int32)
    cu = np.zeros(len(lens) + 1, np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    inp = {"q": _bf(_unit(rng, T, hk, d_)), "k": _bf(_unit(rng, T, hk, d_)),
           "v": _bf(rng.standard_normal((T, hv, d_))),
           "a": rng.uniform(0.5, 1.0, (T, hv)).astype(np.float32),
           "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}
    S0 = (0.3 * rng.standard_normal((len(lens), hv, d_, d_))).astype(np.float32)
    slots = np.arange(len(lens), dtype=np.int32)
    dims = G.make_dims(len(lens), T, max(lens), hk, hv, d_, len(lens), G.GDN_BF16)
    dev = {k: to_dev(v) for k, v in inp.items()}
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    fin = torch.full((len(lens), hv, d_, d_), float("nan"), device="cuda")
    G.gdn_chain_verify(dims, to_dev(cu), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], to_dev(S0),
                       to_dev(slots), out, to_dev(fl), fin, ws=G.new_workspace(dims))
    torch.cuda.synchronize()
    got, gfin = out.cpu().numpy(), fin.cpu().numpy()
    for s, L in enumerate(lens):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = {k: v[lo:hi] for k, v in inp.items()}
        ref, _ = oracle.chain(sl["k"], sl["v"], sl["a"], sl["b"], S0[s], q=sl["q"])
        assert slice_rel_err(got[lo:hi].transpose(1, 0, 2).reshape(hv, -1),
                             ref.transpose(1, 0, 2).reshape(hv, -1)) <= TOL, s
        f = int(fl[s])
        _, ref_fin = oracle.chain(sl["k"][:f], sl["v"][:f], sl["a"][:f], sl["b"][:f], S0[s])
        assert slice_rel_err(gfin[s].reshape(hv, -1), ref_fin.reshape(hv, -1)) <= TOL, s


@pytest.mark.parametrize("nodes", [96, 97, 256])
def test_large_trees(nodes):
    """96 nodes (the largest tree of the node-block kernel), 97 (the smallest the
    coefficient + verify pair takes) and 256 (the per-call maximum)."""
    G = require_gpu()
    rng = np.random.default_rng(22 + nodes)
    hk, hv, d_ = 1, 3, 128
    par = W.random_tree(rng, nodes, 16)
    T = nodes
    inp = {"q": _bf(_unit(rng, T, hk, d_)), "k": _bf(_unit(rng, T, hk, d_)),
           "v": _bf(rng.standard_normal((T, hv, d_))),
           "a": rng.uniform(0.5, 1.0, (T, hv)).astype(np.float32),
           "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}
    S0 = (0.3 * rng.standard_normal((1, hv, d_, d_))).astype(np.float32)
    dims = G.make_dims(1, T, nodes, hk, hv, d_, 1, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in inp.items()}
    cache = to_dev(S0.copy())
    slots = to_dev(np.zeros(1, np.int32))
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    m = int(np.argmax(W.tree_depths(par)))
    G.gdn_tree_plan(dims, to_dev(par), to_dev(np.array([0, T], np.int32)), slots, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache, slots, out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(np.array([m], np.int32)), cache,
                       slots, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    ref = oracle.tree(par, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], S0[0])
    assert slice_rel_err(out.cpu().numpy().transpose(1, 0, 2).reshape(hv, -1),
                         ref.transpose(1, 0, 2).reshape(hv, -1)) <= TOL
    st, _ = oracle.accept_state(par, m, inp["k"], inp["v"], inp["a"], inp["b"], S0[0])
    assert slice_rel_err(cache.cpu().numpy()[0].reshape(hv, -1), st.reshape(hv, -1)) <= TOL


def test_stress_full_size_two_layers():
    """The stress workload at full size in the bench's launch configuration: 64
    sequences x 65-node trees, 48/16 heads, d = 128, one plan serving two
    successive layer calls (verify layer 0, verify layer 1, persist layer 0,
    persist layer 1), each layer with its own inputs and its own state cache
    built from every sequence's prefill.  Every sequence's outputs and persisted
    states on both layers against the oracle; two spare slots per cache stay
    untouched bit for bit."""
    G = require_gpu()
    cfg = W.get_config("stress")
    trees = W.make_trees(cfg)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    acc = W.make_accepts(cfg, trees)
    slots = W.make_slots(cfg)
    hv, d_ = cfg.num_v_heads, cfg.head_dim
    num_slots = cfg.num_slots + 2
    spare = np.setdiff1d(np.arange(num_slots), slots)
    rng = np.random.default_rng(23)
    layers = []
    for layer in (0, 1):
        inp = W.make_layer_inputs(cfg, layer, trees)
        S0 = oracle.initial_states(W.make_prefill(cfg, layer), hv, d_)
        cache = rng.standard_normal((num_slots, hv, d_, d_)).astype(np.float32)
        cache[slots] = S0
        layers.append(dict(inp=inp, S0=S0, cache=cache))
        print("stress layer %d inputs ready" % layer, flush=True)
    dims = G.make_dims(cfg.num_seqs, T, cfg.max_nodes, cfg.num_k_heads, hv, d_, num_slots, G.GDN_BF16)
    ws = G.new_workspace(dims)
    slots_d, acc_d = to_dev(slots), to_dev(acc)
    dev = []
    for L in layers:
        x = {k: to_dev(v) for k, v in L["inp"].items()}
        x["cache"] = to_dev(L["cache"].copy())
        x["out"] = torch.full((T, hv, d_), float("nan"), device="cuda")
        dev.append(x)
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)), slots_d, ws)
    for x in dev:
        G.gdn_tree_verify(dims, x["q"], x["k"], x["v"], x["a"], x["b"], x["cache"], slots_d, x["out"], ws)
    for x in dev:
        G.gdn_tree_persist(dims, x["k"], x["v"], x["a"], x["b"], acc_d, x["cache"], slots_d, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    for layer, (L, x) in enumerate(zip(layers, dev)):
        got = x["out"].cpu().numpy()
        after = x["cache"].cpu().numpy()
        exp = oracle.verify_batch(trees, cu, L["inp"], L["S0"])
        res = oracle.persist_batch(trees, cu, L["inp"], L["S0"], acc)
        worst_o = worst_s = 0.0
        for s in range(cfg.num_seqs):
            lo, hi = int(cu[s]), int(cu[s + 1])
            e = slice_rel_err(got[lo:hi].transpose(1, 0, 2).reshape(hv, -1), exp[lo:hi].transpose(1, 0, 2).reshape(hv, -1))
            assert e <= TOL, (layer, s, e)
            st, _ = res[s]
            es = slice_rel_err(after[slots[s]].reshape(hv, -1), st.reshape(hv, -1))
            assert es <= TOL, (layer, s, es)
            worst_o, worst_s = max(worst_o, e), max(worst_s, es)
        assert np.array_equal(after[spare].view(np.uint32), L["cache"][spare].view(np.uint32))
        print("stress layer %d: verify %.2e, persist %.2e (64 sequences)" % (layer, worst_o, worst_s), flush=True)


def test_many_sequences():
    """4096 sequences of 1-6 nodes in one call (8192 verify and 16384 persist
    workgroups, 4096 plan workgroups each checking every other sequence's slot),
    d=64 with two value heads per key head: sampled sequences against the oracle,
    every output finite, spare slots untouched."""
    G = require_gpu()
    rng = np.random.default_rng(24)
    B, hk, hv, d_ = 4096, 2, 4, 64
    sizes = rng.integers(1, 7, size=B)
    trees = [W.random_tree(rng, int(n), 16) for n in sizes]
    cu = np.zeros(B + 1, np.int32)
    cu[1:] = np.cumsum(sizes)
    T = int(cu[-1])
    inp = {"q": _bf(_unit(rng, T, hk, d_)), "k": _bf(_unit(rng, T, hk, d_)),
           "v": _bf(rng.standard_normal((T, hv, d_))),
           "a": rng.uniform(0.5, 1.0, (T, hv)).astype(np.float32),
           "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}
    n_slots = B + 4
    slots = rng.permutation(n_slots)[:B].astype(np.int32)
    cache = (0.3 * rng.standard_normal((n_slots, hv, d_, d_))).astype(np.float32)
    acc = np.array([rng.integers(0, n) for n in sizes], np.int32)
    dims = G.make_dims(B, T, int(sizes.max()), hk, hv, d_, n_slots, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in inp.items()}
    cache_d = to_dev(cache)
    slots_d = to_dev(slots)
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu), slots_d, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, slots_d, out, ws)
    G.gdn_tree_persist(dims, dev["k"], dev["v"], dev["a"], dev["b"], to_dev(acc), cache_d, slots_d, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    got = out.cpu().numpy()
    assert np.isfinite(got).all()
    after = cache_d.cpu().numpy()
    spare = np.setdiff1d(np.arange(n_slots), slots)
    assert np.array_equal(after[spare].view(np.uint32), cache[spare].view(np.uint32))
    for s in [0, 1, 2047, 4094, 4095] + list(rng.choice(B, 27, replace=False)):
        lo, hi = int(cu[s]), int(cu[s + 1])
        sl = {k: v[lo:hi] for k, v in inp.items()}
        S0 = cache[slots[s]]
        ref = oracle.tree(trees[s], sl["q"], sl["k"], sl["v"], sl["a"], sl["b"], S0)
        assert slice_rel_err(got[lo:hi].transpose(1, 0, 2).reshape(hv, -1),
                             ref.transpose(1, 0, 2).reshape(hv, -1)) <= TOL, s
        st, _ = oracle.accept_state(trees[s], int(acc[s]), sl["k"], sl["v"], sl["a"], sl["b"], S0)
        assert slice_rel_err(after[slots[s]].reshape(hv, -1), st.reshape(hv, -1)) <= TOL, s

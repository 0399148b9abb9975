"""GPU parity of gdn_tree_persist_verify: the persist of one decode step fused
with the verify of the next on one layer.

Bars: every slot the fused call writes holds the same bits as gdn_tree_persist
followed by gdn_tree_verify (the replay arithmetic is shared); outputs within
2e-3 per (sequence, value head) slice of the oracle's verify from the oracle's
persisted states; slots nobody persists stay bitwise untouched; verdicts and
the recorded accepted path as gdn_tree_persist leaves them."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _step(cfg, trees, layer):
    cu = W.cu_from_trees(trees)
    inp = W.make_layer_inputs(cfg, layer, trees)
    return dict(trees=trees, cu=cu, inp=inp)


def _dims(G, cfg, step, num_slots, max_nodes):
    return G.make_dims(cfg.num_seqs, int(step["cu"][-1]), max_nodes, cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim,
                       num_slots, G.GDN_BF16, max_depth=cfg.max_depth)


def _plan(G, dims, step, slots):
    ws = G.new_workspace(dims)
    parent = np.concatenate(step["trees"]).astype(np.int32) if len(step["trees"]) else np.zeros(0, np.int32)
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(step["cu"].astype(np.int32)), to_dev(slots.astype(np.int32)), ws)
    return ws


def _dev_inputs(step):
    return {k: to_dev(v) for k, v in step["inp"].items()}


def _expected_states(prev, S0_by_seq, acc):
    """The oracle's persisted state per sequence (None where nothing is persisted)."""
    res = oracle.persist_batch(prev["trees"], prev["cu"], prev["inp"], S0_by_seq, acc)
    return [r[0] for r in res]


def _run_pair(G, cfg, prev, nxt, slots_prev, slots_next, acc, cache0, num_slots, fused):
    """Either gdn_tree_persist then gdn_tree_verify, or gdn_tree_persist_verify, on
    a copy of cache0; returns outputs, cache and both workspaces."""
    dp = _dims(G, cfg, prev, num_slots, max(int(np.diff(prev["cu"]).max(initial=1)), 1))
    dn = _dims(G, cfg, nxt, num_slots, max(int(np.diff(nxt["cu"]).max(initial=1)), 1))
    wsp = _plan(G, dp, prev, slots_prev)
    wsn = _plan(G, dn, nxt, slots_next)
    xp, xn = _dev_inputs(prev), _dev_inputs(nxt)
    cache = to_dev(cache0.copy())
    T = int(nxt["cu"][-1])
    out = torch.full((max(T, 1), cfg.num_v_heads, cfg.head_dim), float("inf"), device="cuda")[:T]
    acc_d = to_dev(acc.astype(np.int32))
    sl_p, sl_n = to_dev(slots_prev.astype(np.int32)), to_dev(slots_next.astype(np.int32))
    if fused:
        G.gdn_tree_persist_verify(dp, xp["k"], xp["v"], xp["a"], xp["b"], acc_d, wsp, dn, xn["q"], xn["k"], xn["v"],
                                  xn["a"], xn["b"], cache, sl_n, out, wsn)
    else:
        G.gdn_tree_persist(dp, xp["k"], xp["v"], xp["a"], xp["b"], acc_d, cache, sl_p, wsp)
        G.gdn_tree_verify(dn, xn["q"], xn["k"], xn["v"], xn["a"], xn["b"], cache, sl_n, out, wsn)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cache.cpu().numpy(), (dp, wsp), (dn, wsn)


def _check_outputs(cfg, nxt, out, S_by_seq, ok_seqs):
    # sequences left out of the check get a chain of their size for the oracle (a rejected
    # tree is not a tree)
    trees = [t if s in ok_seqs else W.chain_tree(len(t)) for s, t in enumerate(nxt["trees"])]
    exp = oracle.verify_batch(trees, nxt["cu"], nxt["inp"], S_by_seq)
    hv = cfg.num_v_heads
    worst = 0.0
    for s in ok_seqs:
        lo, hi = int(nxt["cu"][s]), int(nxt["cu"][s + 1])
        if hi == lo:
            continue
        e = slice_rel_err(out[lo:hi].transpose(1, 0, 2).reshape(hv, -1), exp[lo:hi].transpose(1, 0, 2).reshape(hv, -1))
        assert e <= TOL, (s, e)
        worst = max(worst, e)
    return worst


@pytest.mark.parametrize("d_", [64, 128])
def test_fused_equals_persist_then_verify_batched(d_):
    """32 sequences of budget-22 DDTrees (48/16 heads) for both steps, new trees and
    inputs in the second, some sequences with nothing accepted; every slot bitwise
    equal to the two-call path, outputs against the oracle, spare slots untouched."""
    G = require_gpu()
    base = W.get_config("batched")
    cfg = dataclasses.replace(base, head_dim=d_)
    cfg2 = dataclasses.replace(cfg, index=cfg.index + 40)
    prev = _step(cfg, W.make_trees(cfg), 0)
    nxt = _step(cfg2, W.make_trees(cfg2), 1)
    slots = W.make_slots(cfg)
    acc = W.make_accepts(cfg, prev["trees"]).copy()
    acc[::5] = -1
    num_slots = cfg.num_slots + 3
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, d_)
    rng = np.random.default_rng(5)
    cache0 = rng.standard_normal((num_slots, cfg.num_v_heads, d_, d_)).astype(np.float32)
    cache0[slots] = S0
    print("fused batched d=%d" % d_, flush=True)
    o_sep, c_sep, (_, wsp_sep), _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, num_slots, False)
    o_fu, c_fu, (dp, wsp), (dn, wsn) = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, num_slots, True)
    assert np.array_equal(c_fu.view(np.uint32), c_sep.view(np.uint32))
    spare = np.setdiff1d(np.arange(num_slots), slots)
    assert np.array_equal(c_fu[spare].view(np.uint32), cache0[spare].view(np.uint32))
    S1 = _expected_states(prev, S0, acc)
    S_new = np.stack([S1[s] if S1[s] is not None else S0[s] for s in range(cfg.num_seqs)])
    for s in range(cfg.num_seqs):
        assert slice_rel_err(c_fu[slots[s]].reshape(cfg.num_v_heads, -1), S_new[s].reshape(cfg.num_v_heads, -1)) <= TOL
    worst = _check_outputs(cfg, nxt, o_fu, S_new, set(range(cfg.num_seqs)))
    # the two paths' outputs differ only by the order the products sum the state's columns
    assert np.abs(o_fu - o_sep).max() <= 1e-4 * np.abs(o_sep).max()
    rc, bad, code = G.gdn_tree_status(wsp)
    assert rc == 0, (rc, bad, code)
    md_f = {k: v.cpu().numpy() for k, v in G.read_metadata(dp, wsp).items()}
    md_s = {k: v.cpu().numpy() for k, v in G.read_metadata(dp, wsp_sep).items()}
    live = acc >= 0
    assert np.array_equal(md_f["path_len"][live], md_s["path_len"][live])
    assert np.array_equal(md_f["path"][live], md_s["path"][live])
    print("fused batched d=%d: worst output error %.2e" % (d_, worst), flush=True)


def _ragged_case(d_=64):
    cfg = dataclasses.replace(W.get_config("batched"), num_seqs=6, num_k_heads=2, num_v_heads=4, head_dim=d_,
                              num_slots=8, index=77)
    rng = np.random.default_rng(31)
    sizes_p = [5, 23, 1, 17, 9, 32]
    sizes_n = [12, 0, 7, 3, 32, 20]
    trees_p = [W.random_tree(rng, n, 16) for n in sizes_p]
    trees_n = [W.random_tree(rng, n, 16) for n in sizes_n]
    return cfg, trees_p, trees_n


def test_fused_ragged_empty_rejected_and_skipped():
    """Six sequences at d = 64, two value heads per key head: a skipped accept, an
    empty new tree, a rejected new tree (its sequence is still persisted: no other
    verified sequence reads its slot), ragged sizes up to 32 nodes, two spare slots."""
    G = require_gpu()
    cfg, trees_p, trees_n = _ragged_case()
    trees_n[3] = np.array([-1, 0, 2], dtype=np.int32)  # node 2 is its own parent: rejected
    slots = np.array([3, 0, 5, 1, 4, 2])
    acc = np.array([2, -1, 0, 16, 4, 31])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    num_slots = cfg.num_slots
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    cache0 = np.random.default_rng(8).standard_normal((num_slots, cfg.num_v_heads, cfg.head_dim,
                                                      cfg.head_dim)).astype(np.float32)
    cache0[slots] = S0
    print("fused ragged", flush=True)
    o_sep, c_sep, _, _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, num_slots, False)
    o_fu, c_fu, (dp, wsp), (dn, wsn) = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, num_slots, True)
    assert np.array_equal(c_fu.view(np.uint32), c_sep.view(np.uint32))
    assert np.array_equal(c_fu[[6, 7]].view(np.uint32), cache0[[6, 7]].view(np.uint32))
    S1 = _expected_states(prev, S0, acc)
    S_new = np.stack([S1[s] if S1[s] is not None else S0[s] for s in range(cfg.num_seqs)])
    _check_outputs(cfg, nxt, o_fu, S_new, {0, 2, 4, 5})
    lo, hi = int(nxt["cu"][3]), int(nxt["cu"][4])
    assert np.isnan(o_fu[lo:hi]).all()
    assert G.gdn_tree_status(wsp)[0] == 0
    rc, bad, code = G.gdn_tree_status(wsn)
    assert (rc, bad, code) == (-6, 3, 4)  # GDN_ERR_TREE: sequence 3, GDN_SEQ_BAD_PARENT


def test_fused_slot_clash_is_not_persisted():
    """Two sequences swap slots between the steps: each would write the slot the
    other verifies from, so neither is persisted (both marked NOT_PERSISTED, both
    slots untouched) and each is verified from the committed state in its new slot;
    the other sequences are persisted and verified as usual."""
    G = require_gpu()
    cfg, trees_p, trees_n = _ragged_case()
    trees_n[1] = W.random_tree(np.random.default_rng(4), 6, 16)
    slots_p = np.array([3, 0, 5, 1, 4, 2])
    slots_n = np.array([0, 3, 5, 1, 4, 2])
    acc = np.array([2, 11, 0, 16, 4, 31])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    num_slots = cfg.num_slots
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    cache0 = np.random.default_rng(9).standard_normal((num_slots, cfg.num_v_heads, cfg.head_dim,
                                                      cfg.head_dim)).astype(np.float32)
    cache0[slots_p] = S0
    print("fused clash", flush=True)
    o_fu, c_fu, (dp, wsp), _ = _run_pair(G, cfg, prev, nxt, slots_p, slots_n, acc, cache0, num_slots, True)
    for sl in (0, 3, 6, 7):
        assert np.array_equal(c_fu[sl].view(np.uint32), cache0[sl].view(np.uint32)), sl
    S1 = _expected_states(prev, S0, acc)
    for s in (2, 3, 4, 5):
        assert slice_rel_err(c_fu[slots_p[s]].reshape(cfg.num_v_heads, -1),
                             S1[s].reshape(cfg.num_v_heads, -1)) <= TOL
    # the state each sequence is verified from: its new slot after the call
    S_ver = np.stack([c_fu[slots_n[s]].astype(np.float64) if s in (0, 1) else S1[s] for s in range(cfg.num_seqs)])
    _check_outputs(cfg, nxt, o_fu, S_ver, set(range(cfg.num_seqs)))
    md = {k: v.cpu().numpy() for k, v in G.read_metadata(dp, wsp).items()}
    assert list(md["seq_status"]) == [7, 7, 0, 0, 0, 0]
    assert G.gdn_tree_status(wsp)[1:] == (0, 7)


def test_fused_rejects_a_workspace_planned_for_other_dims():
    """A previous-step workspace planned for another node count: nothing is
    written (cache and outputs untouched) and that workspace reports misuse."""
    G = require_gpu()
    cfg, trees_p, trees_n = _ragged_case()
    slots = np.array([3, 0, 5, 1, 4, 2])
    acc = np.array([2, -1, 0, 16, 4, 31])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    cache0 = np.random.default_rng(10).standard_normal((cfg.num_slots, cfg.num_v_heads, cfg.head_dim,
                                                       cfg.head_dim)).astype(np.float32)
    dp = _dims(G, cfg, prev, cfg.num_slots, 32)
    dn = _dims(G, cfg, nxt, cfg.num_slots, 32)
    wsp = _plan(G, dp, prev, slots)
    wsn = _plan(G, dn, nxt, slots)
    dp_other = _dims(G, cfg, prev, cfg.num_slots, 24)  # the plan was made for max_nodes 32
    xp, xn = _dev_inputs(prev), _dev_inputs(nxt)
    cache = to_dev(cache0.copy())
    out = torch.full((int(nxt["cu"][-1]), cfg.num_v_heads, cfg.head_dim), 7.0, device="cuda")
    G.gdn_tree_persist_verify(dp_other, xp["k"], xp["v"], xp["a"], xp["b"], to_dev(acc.astype(np.int32)), wsp, dn,
                              xn["q"], xn["k"], xn["v"], xn["a"], xn["b"], cache, to_dev(slots.astype(np.int32)), out,
                              wsn)
    torch.cuda.synchronize()
    assert np.array_equal(cache.cpu().numpy().view(np.uint32), cache0.view(np.uint32))
    assert (out.cpu().numpy() == 7.0).all()
    assert G.gdn_tree_status(wsp)[0] == -4  # GDN_ERR_WORKSPACE


def test_fused_graph_replays_match_eager():
    """The fused call captured in a HIP graph: four replays (eager work and a
    synchronization between them) each equal to the eager call bit for bit."""
    G = require_gpu()
    cfg, trees_p, trees_n = _ragged_case(128)
    slots = np.array([3, 0, 5, 1, 4, 2])
    acc = np.array([2, -1, 0, 16, 4, 31])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    cache0 = np.random.default_rng(12).standard_normal((cfg.num_slots, cfg.num_v_heads, cfg.head_dim,
                                                       cfg.head_dim)).astype(np.float32)
    dp = _dims(G, cfg, prev, cfg.num_slots, 32)
    dn = _dims(G, cfg, nxt, cfg.num_slots, 32)
    wsp = _plan(G, dp, prev, slots)
    wsn = _plan(G, dn, nxt, slots)
    xp, xn = _dev_inputs(prev), _dev_inputs(nxt)
    acc_d, sl_d = to_dev(acc.astype(np.int32)), to_dev(slots.astype(np.int32))
    src = to_dev(cache0.copy())
    cache = src.clone()
    out = torch.zeros((int(nxt["cu"][-1]), cfg.num_v_heads, cfg.head_dim), device="cuda")

    def call():
        G.gdn_tree_persist_verify(dp, xp["k"], xp["v"], xp["a"], xp["b"], acc_d, wsp, dn, xn["q"], xn["k"], xn["v"],
                                  xn["a"], xn["b"], cache, sl_d, out, wsn)

    call()
    torch.cuda.synchronize()
    ref_out, ref_cache = out.clone(), cache.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cache.copy_(src)
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for _ in range(4):
        cache.copy_(src)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out)
        assert torch.equal(cache.view(torch.int32), ref_cache.view(torch.int32))


@pytest.mark.parametrize("shape", [("40 nodes", 128, "bf16", 40), ("fp32 inputs", 64, "f32", 20),
                                   ("d = 32", 32, "bf16", 20)])
def test_fused_entry_point_falls_back_to_the_two_calls(shape):
    """Shapes the fused kernel does not take (trees over 32 nodes, fp32 inputs, a head
    dim of 32) run gdn_tree_persist then gdn_tree_verify inside the call: outputs and
    every slot bit for bit those of the two calls, and within 2e-3 of the oracle."""
    G = require_gpu()
    label, d_, dt, nmax = shape
    cfg = dataclasses.replace(W.get_config("batched"), num_seqs=4, num_k_heads=2, num_v_heads=4, head_dim=d_,
                              num_slots=6, index=91, dtype=dt)
    rng = np.random.default_rng(17)
    trees_p = [W.random_tree(rng, n, 16) for n in (nmax, 7, nmax - 3, 12)]
    trees_n = [W.random_tree(rng, n, 16) for n in (9, nmax, 5, nmax - 1)]
    slots = np.array([4, 1, 0, 3])
    acc = np.array([nmax - 1, 3, -1, 11])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, d_)
    cache0 = np.random.default_rng(18).standard_normal((cfg.num_slots, cfg.num_v_heads, d_, d_)).astype(np.float32)
    cache0[slots] = S0
    qkv = G.GDN_F32 if dt == "f32" else G.GDN_BF16

    def run(fused):
        dp = G.make_dims(cfg.num_seqs, int(prev["cu"][-1]), nmax, cfg.num_k_heads, cfg.num_v_heads, d_,
                         cfg.num_slots, qkv)
        dn = G.make_dims(cfg.num_seqs, int(nxt["cu"][-1]), nmax, cfg.num_k_heads, cfg.num_v_heads, d_,
                         cfg.num_slots, qkv)
        wsp, wsn = _plan(G, dp, prev, slots), _plan(G, dn, nxt, slots)
        xp, xn = _dev_inputs(prev), _dev_inputs(nxt)
        cache = to_dev(cache0.copy())
        out = torch.zeros((int(nxt["cu"][-1]), cfg.num_v_heads, d_), device="cuda")
        acc_d, sl = to_dev(acc.astype(np.int32)), to_dev(slots.astype(np.int32))
        if fused:
            G.gdn_tree_persist_verify(dp, xp["k"], xp["v"], xp["a"], xp["b"], acc_d, wsp, dn, xn["q"], xn["k"],
                                      xn["v"], xn["a"], xn["b"], cache, sl, out, wsn)
        else:
            G.gdn_tree_persist(dp, xp["k"], xp["v"], xp["a"], xp["b"], acc_d, cache, sl, wsp)
            G.gdn_tree_verify(dn, xn["q"], xn["k"], xn["v"], xn["a"], xn["b"], cache, sl, out, wsn)
        torch.cuda.synchronize()
        assert G.gdn_tree_status(wsp)[0] == 0 and G.gdn_tree_status(wsn)[0] == 0
        return out.cpu().numpy(), cache.cpu().numpy()

    print("fused fallback:", label, flush=True)
    o_f, c_f = run(True)
    o_s, c_s = run(False)
    assert np.array_equal(o_f.view(np.uint32), o_s.view(np.uint32))
    assert np.array_equal(c_f.view(np.uint32), c_s.view(np.uint32))
    S1 = _expected_states(prev, S0, acc)
    S_new = np.stack([S1[s] if S1[s] is not None else S0[s] for s in range(cfg.num_seqs)])
    _check_outputs(cfg, nxt, o_f, S_new, set(range(cfg.num_seqs)))


@pytest.mark.parametrize("seed", range(6))
def test_fused_seeded_sweep(seed):
    """Seeded shapes for the fused kernel: 1-40 sequences, trees of 1-32 nodes (random
    and chains), 1-4 value heads per key head, d 64 or 128, accepted nodes anywhere or
    -1, a slot permutation with spare slots; slots and outputs bitwise equal to the two
    calls' where the kernels share arithmetic (slots), outputs against the oracle."""
    G = require_gpu()
    rng = np.random.default_rng(1000 + seed)
    d_ = int(rng.choice([64, 128]))
    hk = int(rng.integers(1, 3))
    ratio = int(rng.integers(1, 5))
    B = int(rng.integers(1, 41))
    cfg = dataclasses.replace(W.get_config("batched"), num_seqs=B, num_k_heads=hk, num_v_heads=hk * ratio,
                              head_dim=d_, num_slots=B + 2, index=200 + seed)

    def tree():
        n = int(rng.integers(1, 33))
        return W.chain_tree(min(n, 16)) if rng.random() < 0.2 else W.random_tree(rng, n, 16)

    trees_p = [tree() for _ in range(B)]
    trees_n = [tree() for _ in range(B)]
    acc = np.array([int(rng.integers(-1, len(t))) for t in trees_p])
    slots = rng.permutation(B + 2)[:B]
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, d_)
    cache0 = rng.standard_normal((B + 2, cfg.num_v_heads, d_, d_)).astype(np.float32)
    cache0[slots] = S0
    print("fused sweep seed %d: B=%d hk=%d hv=%d d=%d" % (seed, B, hk, hk * ratio, d_), flush=True)
    o_s, c_s, _, _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, B + 2, False)
    o_f, c_f, (_, wsp), _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, B + 2, True)
    assert np.array_equal(c_f.view(np.uint32), c_s.view(np.uint32))
    assert G.gdn_tree_status(wsp)[0] == 0
    S1 = _expected_states(prev, S0, acc)
    S_new = np.stack([S1[s] if S1[s] is not None else S0[s] for s in range(B)])
    _check_outputs(cfg, nxt, o_f, S_new, set(range(B)))


def test_fused_off_path_inputs_leave_results_bitwise():
    """P-anc through the fused call: perturbing the previous step's inputs off each
    accepted path leaves every persisted slot unchanged bit for bit, and perturbing
    the new trees' leaves (no node's ancestors) leaves every other node's outputs
    unchanged bit for bit (32 sequences of 23-node DDTrees, 48/16 heads, d = 128)."""
    G = require_gpu()
    cfg = W.get_config("batched")
    cfg2 = dataclasses.replace(cfg, index=cfg.index + 41)
    prev = _step(cfg, W.make_trees(cfg), 0)
    nxt = _step(cfg2, W.make_trees(cfg2), 1)
    slots = W.make_slots(cfg)
    acc = W.make_accepts(cfg, prev["trees"])
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    cache0 = np.zeros((cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim), np.float32)
    cache0[slots] = S0
    rng = np.random.default_rng(77)

    def perturb(step, rows):
        out = dict(step)
        inp = {k: v.copy() for k, v in step["inp"].items()}
        for k, v in inp.items():
            if v.dtype == np.uint16:  # bf16 bits: flip low mantissa bits
                v[rows] ^= rng.integers(1, 64, size=v[rows].shape, dtype=np.uint16)
            else:
                v[rows] = v[rows] * np.float32(0.5) + np.float32(0.25)
        out["inp"] = inp
        return out

    off_path, leaves = [], []
    for s in range(cfg.num_seqs):
        par, lo = prev["trees"][s], int(prev["cu"][s])
        on, m = set(), int(acc[s])
        while m >= 0:
            on.add(m)
            m = int(par[m])
        off_path += [lo + i for i in range(len(par)) if i not in on]
        parn, lon = nxt["trees"][s], int(nxt["cu"][s])
        has_child = set(int(p) for p in parn if p >= 0)
        leaves += [lon + i for i in range(len(parn)) if i not in has_child]
    off_path, leaves = np.array(off_path), np.array(leaves)
    print("fused P-anc: %d off-path nodes, %d leaves" % (len(off_path), len(leaves)), flush=True)
    o_a, c_a, _, _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, cfg.num_slots, True)
    o_b, c_b, _, _ = _run_pair(G, cfg, perturb(prev, off_path), perturb(nxt, leaves), slots, slots, acc, cache0,
                               cfg.num_slots, True)
    assert np.array_equal(c_a.view(np.uint32), c_b.view(np.uint32))
    keep = np.setdiff1d(np.arange(o_a.shape[0]), leaves)
    assert np.array_equal(o_a[keep].view(np.uint32), o_b[keep].view(np.uint32))
    assert not np.array_equal(o_a[leaves], o_b[leaves])  # the perturbation reached the leaves


def test_fused_rejected_previous_tree_and_bad_accept():
    """A previous-step tree the plan rejected is not persisted, and an accepted node
    out of range marks GDN_SEQ_BAD_ACCEPT and persists nothing, exactly as
    gdn_tree_persist does; both sequences are still verified from their committed
    state.  Slots and verdicts equal to the two calls', outputs against the oracle."""
    G = require_gpu()
    cfg, trees_p, trees_n = _ragged_case(128)
    trees_p[2] = np.array([-1, 0, 5], dtype=np.int32)  # parent 5 outside the 3-node tree: rejected
    slots = np.array([3, 0, 5, 1, 4, 2])
    acc = np.array([2, 40, 0, 16, 4, 31])  # sequence 1's 23-node tree has no node 40
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    cache0 = np.random.default_rng(21).standard_normal((cfg.num_slots, cfg.num_v_heads, cfg.head_dim,
                                                       cfg.head_dim)).astype(np.float32)
    cache0[slots] = S0
    print("fused rejected previous tree, bad accept", flush=True)
    o_s, c_s, (dp, wsp_s), _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, cfg.num_slots, False)
    o_f, c_f, (_, wsp_f), _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, cfg.num_slots, True)
    assert np.array_equal(c_f.view(np.uint32), c_s.view(np.uint32))
    for sl in (slots[1], slots[2]):
        assert np.array_equal(c_f[sl].view(np.uint32), cache0[sl].view(np.uint32))
    st_f = G.read_metadata(dp, wsp_f)["seq_status"].cpu().numpy()
    st_s = G.read_metadata(dp, wsp_s)["seq_status"].cpu().numpy()
    assert np.array_equal(st_f, st_s) and st_f[1] == 6 and st_f[2] == 4, (st_f, st_s)
    acc_ok = acc.copy()
    acc_ok[[1, 2]] = -1
    S1 = _expected_states(dict(prev, trees=[t if s != 2 else W.chain_tree(3) for s, t in enumerate(prev["trees"])]),
                          S0, acc_ok)
    S_new = np.stack([S1[s] if S1[s] is not None else S0[s] for s in range(cfg.num_seqs)])
    _check_outputs(cfg, nxt, o_f, S_new, set(range(cfg.num_seqs)) - {1})  # sequence 1's new tree is empty


def test_fused_after_a_step_with_large_trees():
    """The fused kernel is chosen by the new step's trees (at most 32 nodes); the
    previous step's may be larger (here 60-200 nodes: its accepted path is still at
    most 16 nodes).  Slots bitwise equal to the two calls, outputs against the oracle."""
    G = require_gpu()
    cfg = dataclasses.replace(W.get_config("batched"), num_seqs=5, num_k_heads=2, num_v_heads=6, head_dim=128,
                              num_slots=7, index=131)
    rng = np.random.default_rng(41)
    trees_p = [W.random_tree(rng, n, 16) for n in (60, 200, 97, 128, 75)]
    trees_n = [W.random_tree(rng, n, 16) for n in (32, 9, 23, 1, 30)]
    slots = np.array([6, 2, 0, 4, 3])
    acc = np.array([int(rng.integers(0, len(t))) for t in trees_p])
    prev = _step(cfg, trees_p, 0)
    nxt = _step(cfg, trees_n, 1)
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    cache0 = rng.standard_normal((cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim)).astype(np.float32)
    cache0[slots] = S0
    print("fused after large trees", flush=True)
    o_s, c_s, _, _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, cfg.num_slots, False)
    o_f, c_f, (_, wsp), _ = _run_pair(G, cfg, prev, nxt, slots, slots, acc, cache0, cfg.num_slots, True)
    assert np.array_equal(c_f.view(np.uint32), c_s.view(np.uint32))
    assert G.gdn_tree_status(wsp)[0] == 0
    S1 = _expected_states(prev, S0, acc)
    _check_outputs(cfg, nxt, o_f, np.stack(S1), set(range(cfg.num_seqs)))


def test_deferred_persist_decode_loop_over_four_steps():
    """The decode loop the fused call is for, on one layer over four steps with new
    trees, inputs and accepted nodes each step: step 0 verify; steps 1-3 fused (persist
    of the step before + verify); a final plain persist.  Every step's outputs and the
    final cache against the oracle's sequential loop (verify then persist per step),
    and the final cache bitwise equal to the same loop run with the two calls."""
    G = require_gpu()
    base = dataclasses.replace(W.get_config("batched"), num_seqs=8, num_slots=10)
    steps = [dataclasses.replace(base, index=300 + t) for t in range(4)]
    trees = [W.make_trees(c) for c in steps]
    data = [_step(c, tr, t) for t, (c, tr) in enumerate(zip(steps, trees))]
    accs = [W.make_accepts(c, tr) for c, tr in zip(steps, trees)]
    accs[1] = accs[1].copy()
    accs[1][3] = -1  # a sequence that accepts nothing in one step
    slots = W.make_slots(base)
    S0 = oracle.initial_states(W.make_prefill(base, 0), base.num_v_heads, base.head_dim)
    cache0 = np.random.default_rng(61).standard_normal((base.num_slots, base.num_v_heads, base.head_dim,
                                                       base.head_dim)).astype(np.float32)
    cache0[slots] = S0
    # the oracle's loop
    S = S0.astype(np.float64)
    exp_out = []
    for t in range(4):
        exp_out.append(oracle.verify_batch(data[t]["trees"], data[t]["cu"], data[t]["inp"], S))
        st = _expected_states(data[t], S, accs[t])
        S = np.stack([st[s] if st[s] is not None else S[s] for s in range(base.num_seqs)])

    def run(fused):
        dims = [_dims(G, base, d, base.num_slots, 32) for d in data]
        wss = [_plan(G, dm, d, slots) for dm, d in zip(dims, data)]
        xs = [_dev_inputs(d) for d in data]
        acc_d = [to_dev(a.astype(np.int32)) for a in accs]
        sl = to_dev(slots.astype(np.int32))
        cache = to_dev(cache0.copy())
        outs = []
        for t in range(4):
            out = torch.zeros((int(data[t]["cu"][-1]), base.num_v_heads, base.head_dim), device="cuda")
            x = xs[t]
            if t == 0 or not fused:
                if t > 0:
                    p = xs[t - 1]
                    G.gdn_tree_persist(dims[t - 1], p["k"], p["v"], p["a"], p["b"], acc_d[t - 1], cache, sl, wss[t - 1])
                G.gdn_tree_verify(dims[t], x["q"], x["k"], x["v"], x["a"], x["b"], cache, sl, out, wss[t])
            else:
                p = xs[t - 1]
                G.gdn_tree_persist_verify(dims[t - 1], p["k"], p["v"], p["a"], p["b"], acc_d[t - 1], wss[t - 1], dims[t],
                                          x["q"], x["k"], x["v"], x["a"], x["b"], cache, sl, out, wss[t])
            outs.append(out)
        p = xs[3]
        G.gdn_tree_persist(dims[3], p["k"], p["v"], p["a"], p["b"], acc_d[3], cache, sl, wss[3])
        torch.cuda.synchronize()
        for w_ in wss:
            assert G.gdn_tree_status(w_)[0] == 0
        return [o.cpu().numpy() for o in outs], cache.cpu().numpy()

    print("deferred-persist decode loop", flush=True)
    outs_f, cache_f = run(True)
    outs_s, cache_s = run(False)
    assert np.array_equal(cache_f.view(np.uint32), cache_s.view(np.uint32))
    for t in range(4):
        hv = base.num_v_heads
        for s in range(base.num_seqs):
            lo, hi = int(data[t]["cu"][s]), int(data[t]["cu"][s + 1])
            e = slice_rel_err(outs_f[t][lo:hi].transpose(1, 0, 2).reshape(hv, -1),
                              exp_out[t][lo:hi].transpose(1, 0, 2).reshape(hv, -1))
            assert e <= TOL, (t, s, e)
    for s in range(base.num_seqs):
        assert slice_rel_err(cache_f[slots[s]].reshape(base.num_v_heads, -1),
                             S[s].reshape(base.num_v_heads, -1)) <= TOL, s

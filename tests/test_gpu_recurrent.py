"""The per-node recurrent kernels on the bf16 / head-dim-128 workloads, where
the library would otherwise pick the matrix-core kernels (forced with
GDN_KERNEL_PATH=recurrent): oracle parity, chain == chain-shaped tree bit for
bit, and persisted state == the chain kernel's final state bit for bit."""
import numpy as np
import pytest
import torch

from gpu_support import TOL, device_case, host_case, require_gpu, run_step, slice_rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture
def recurrent(monkeypatch):
    monkeypatch.setenv("GDN_KERNEL_PATH", "recurrent")
    yield


def _out_err(case, out):
    cfg = case["cfg"]
    worst = 0.0
    for s in range(cfg.num_seqs):
        lo, hi = int(case["cu"][s]), int(case["cu"][s + 1])
        x = out[lo:hi].transpose(1, 0, 2).reshape(cfg.num_v_heads, -1)
        r = case["exp_out"][lo:hi].transpose(1, 0, 2).reshape(cfg.num_v_heads, -1)
        worst = max(worst, slice_rel_err(x, r))
    return worst


@pytest.mark.parametrize("name", ["chain", "ddtree22", "batched"])
def test_recurrent_parity(name, recurrent):
    G = require_gpu()
    case = host_case(name)
    d = device_case(G, case)
    print("recurrent path", name, flush=True)
    run_step(G, d, persist=True)
    assert _out_err(case, d["out"].cpu().numpy()) <= TOL
    cache = d["cache"].cpu().numpy()
    for s in range(case["cfg"].num_seqs):
        st, _ = case["exp_persist"][s]
        got = cache[int(case["slots"][s])]
        assert slice_rel_err(got.reshape(case["cfg"].num_v_heads, -1), st.reshape(case["cfg"].num_v_heads, -1)) <= TOL


def test_recurrent_chain_tree_bitwise(recurrent):
    G = require_gpu()
    case = host_case("chain")
    d = device_case(G, case)
    run_step(G, d, persist=False)
    tree_out = d["out"].clone()
    dims = d["dims"]
    n = int(case["cu"][-1])
    out = torch.full_like(tree_out, float("nan"))
    fin = torch.full((1, dims.num_v_heads, dims.head_dim, dims.head_dim), float("nan"), device="cuda")
    flen = torch.tensor([int(case["acc"][0]) + 1], dtype=torch.int32, device="cuda")
    G.gdn_chain_verify(dims, d["cu"], d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], d["slots"], out, flen,
                       fin, ws=G.new_workspace(dims))
    torch.cuda.synchronize()
    assert torch.equal(tree_out.view(torch.int32), out.view(torch.int32))
    G.gdn_tree_persist(dims, d["k"], d["v"], d["a"], d["b"], d["acc"], d["cache"], d["slots"], d["ws"])
    torch.cuda.synchronize()
    slot = int(case["slots"][0])
    assert torch.equal(d["cache"][slot].view(torch.int32), fin[0].view(torch.int32))
    assert n == 16


def test_recurrent_tree_fills_the_state_stack(recurrent):
    """Trees whose heavy-last preorder fills the state stack to its bound (a
    complete binary tree of 63 nodes: five nested pushes, the bound for 63
    nodes), a complete ternary tree, a relabelled copy of the binary tree and a
    random recursive tree, each accepted at a deepest leaf: outputs and
    persisted states against the oracle, spare slots untouched."""
    import dataclasses

    import oracle
    import workloads as W
    from oracle import plan as oplan

    G = require_gpu()
    cfg = dataclasses.replace(W.get_config("batched"), num_seqs=4, num_slots=6, tree=("random", 63, 16))
    binary = np.array([-1] + [(i - 1) // 2 for i in range(1, 63)], np.int32)
    ternary = np.array([-1] + [(i - 1) // 3 for i in range(1, 40)], np.int32)
    rng = np.random.default_rng(5)
    perm = rng.permutation(63)
    relabelled = np.empty(63, np.int32)
    relabelled[perm] = np.where(binary >= 0, perm[np.maximum(binary, 0)], -1)
    rand = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, 63)], np.int32)
    trees = [binary, ternary, relabelled, rand]
    plans = [oplan.plan_tree(t) for t in trees]
    assert plans[0]["max_stack"] == oplan.stack_bound(63) == 5
    assert all(int(np.max(p["depth"])) <= cfg.max_depth for p in plans)
    cu = W.cu_from_trees(trees)
    inp = W.make_layer_inputs(cfg, 0, trees)
    S0 = oracle.initial_states(W.make_prefill(cfg, 0), cfg.num_v_heads, cfg.head_dim)
    slots = W.make_slots(cfg)
    acc = np.array([62, 39, int(perm[62]), 62], np.int32)  # a deepest leaf of each tree
    cache = np.random.default_rng(99).standard_normal(
        (cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim)).astype(np.float32)
    for s in range(cfg.num_seqs):
        cache[slots[s]] = S0[s]
    case = dict(cfg=cfg, trees=trees, cu=cu, inp=inp, S0=S0, slots=slots, acc=acc, cache=cache,
                num_slots=cfg.num_slots, exp_out=oracle.verify_batch(trees, cu, inp, S0),
                exp_persist=oracle.persist_batch(trees, cu, inp, S0, acc))
    d = device_case(G, case)
    print("recurrent path, full state stack", flush=True)
    run_step(G, d, persist=True)
    assert G.gdn_tree_status(d["ws"])[0] == 0
    assert _out_err(case, d["out"].cpu().numpy()) <= TOL
    got = d["cache"].cpu().numpy()
    for s in range(cfg.num_seqs):
        st, _ = case["exp_persist"][s]
        x = got[int(slots[s])].reshape(cfg.num_v_heads, -1)
        assert slice_rel_err(x, st.reshape(cfg.num_v_heads, -1)) <= TOL, s
    spare = sorted(set(range(cfg.num_slots)) - {int(x) for x in slots})
    assert spare and np.array_equal(got[spare].view(np.uint32), cache[spare].view(np.uint32))

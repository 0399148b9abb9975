"""The per-node-state path kept for comparison (gdn_tree_verify_store +
gdn_tree_persist_copy): outputs, stored fp16 node states and the committed
state against the oracle, to the 2e-3 slice bar (fp16 storage rounds each
value by at most 2^-11 relative)."""
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_support import TOL, device_case, host_case, require_gpu, slice_rel_err

pytestmark = pytest.mark.gpu


def _store_step(G, d, T, hv, dd):
    node_states = torch.full((T, hv, dd, dd), 3.0, dtype=torch.float16, device="cuda")
    G.gdn_tree_plan(d["dims"], d["parent"], d["cu"], d["slots"], d["ws"])
    G.gdn_tree_verify_store(d["dims"], d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], d["slots"], d["out"],
                            node_states, d["ws"])
    return node_states


@pytest.mark.parametrize("name", ["tiny", "ddtree22", "batched"])
def test_store_outputs_states_and_copy_persist(name):
    G = require_gpu()
    case = host_case(name)
    cfg = case["cfg"]
    d = device_case(G, case)
    T, hv, dd = int(case["cu"][-1]), cfg.num_v_heads, cfg.head_dim
    ns = _store_step(G, d, T, hv, dd)
    torch.cuda.synchronize()
    out = d["out"].cpu().numpy()
    worst = 0.0
    for s in range(cfg.num_seqs):
        lo, hi = int(case["cu"][s]), int(case["cu"][s + 1])
        exp = case["exp_out"][lo:hi]
        for h in range(hv):
            worst = max(worst, slice_rel_err(out[lo:hi, h].reshape(1, -1), exp[:, h].reshape(1, -1)))
    assert worst <= TOL, worst
    # every node's stored state against the oracle's node states (one sequence's worth per check)
    states = ns.float().cpu().numpy()
    for s in range(min(cfg.num_seqs, 4)):
        lo, hi = int(case["cu"][s]), int(case["cu"][s + 1])
        sl = {k: v[lo:hi] for k, v in case["inp"].items()}
        _, st = oracle.tree(case["trees"][s], sl["q"], sl["k"], sl["v"], sl["a"], sl["b"], case["S0"][s],
                            return_states=True)
        err = slice_rel_err(states[lo:hi].reshape(hi - lo, hv, -1).reshape(-1, dd * dd),
                            st.reshape(-1, dd * dd))
        assert err <= TOL, (s, err)
    # commit by copy
    G.gdn_tree_persist_copy(d["dims"], d["acc"], ns, d["cache"], d["slots"], d["ws"])
    rc = G.gdn_tree_status(d["ws"])
    assert rc[0] == 0, rc
    cache = d["cache"].cpu().numpy()
    touched = set()
    for s in range(cfg.num_seqs):
        st, _ = case["exp_persist"][s]
        slot = int(case["slots"][s])
        touched.add(slot)
        assert slice_rel_err(cache[slot].reshape(hv, -1), st.reshape(hv, -1)) <= TOL
    for slot in range(case["num_slots"]):
        if slot not in touched:
            assert np.array_equal(cache[slot].view(np.uint32), case["cache"][slot].view(np.uint32))


def test_store_keeps_outputs_of_the_recurrent_verify():
    """Storing adds no arithmetic: outputs equal the recurrent verify's bit for bit."""
    G = require_gpu()
    case = host_case("ddtree22")
    cfg = case["cfg"]
    d = device_case(G, case)
    T = int(case["cu"][-1])
    _store_step(G, d, T, cfg.num_v_heads, cfg.head_dim)
    torch.cuda.synchronize()
    a = d["out"].cpu().numpy().copy()
    os.environ["GDN_KERNEL_PATH"] = "recurrent"
    try:
        G.gdn_tree_verify(d["dims"], d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], d["slots"], d["out"], d["ws"])
        torch.cuda.synchronize()
    finally:
        del os.environ["GDN_KERNEL_PATH"]
    assert np.array_equal(a.view(np.uint32), d["out"].cpu().numpy().view(np.uint32))


def test_copy_persist_rejects_bad_accepted_node():
    G = require_gpu()
    case = host_case("ddtree22")
    cfg = case["cfg"]
    d = device_case(G, case)
    T = int(case["cu"][-1])
    ns = _store_step(G, d, T, cfg.num_v_heads, cfg.head_dim)
    before = d["cache"].cpu().numpy().copy()
    bad = torch.tensor([T + 5], dtype=torch.int32, device="cuda")
    G.gdn_tree_persist_copy(d["dims"], bad, ns, d["cache"], d["slots"], d["ws"])
    rc, seq, code = G.gdn_tree_status(d["ws"])
    assert rc == G.GdnError(-6, "").code and seq == 0 and code == 6
    assert np.array_equal(before.view(np.uint32), d["cache"].cpu().numpy().view(np.uint32))

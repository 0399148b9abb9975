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

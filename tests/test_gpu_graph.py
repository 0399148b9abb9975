"""Decode steps captured in a HIP graph (plan -> verify -> persist, two
consecutive steps per graph, as the bench replays a cycle of steps): every
replay, with eager work and synchronizations in between, must reproduce the
eager steps bit for bit."""
import numpy as np
import pytest
import torch

from gpu_support import device_case, host_case, require_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["ddtree22", "batched"])
def test_graph_replays_match_eager(name):
    G = require_gpu()
    case = host_case(name)
    d = device_case(G, case)
    pristine = d["cache"].clone()

    def step():
        G.gdn_tree_plan(d["dims"], d["parent"], d["cu"], d["slots"], d["ws"])
        G.gdn_tree_verify(d["dims"], d["q"], d["k"], d["v"], d["a"], d["b"], d["cache"], d["slots"], d["out"],
                          d["ws"])
        G.gdn_tree_persist(d["dims"], d["k"], d["v"], d["a"], d["b"], d["acc"], d["cache"], d["slots"], d["ws"])

    step()
    step()  # the second step verifies against the first one's persisted states
    torch.cuda.synchronize()
    want_out = d["out"].cpu().numpy().copy()
    want_cache = d["cache"].cpu().numpy().copy()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        d["cache"].copy_(pristine)
        step()  # warm the side stream (attribute setup, code objects) before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
        step()
    for rep in range(4):
        d["cache"].copy_(pristine)
        d["out"].fill_(float("nan"))
        d["ws"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(d["out"].cpu().numpy().view(np.uint32), want_out.view(np.uint32)), rep
        assert np.array_equal(d["cache"].cpu().numpy().view(np.uint32), want_cache.view(np.uint32)), rep
        _ = torch.randn(1000, device="cuda").sum().item()  # unrelated eager work between replays

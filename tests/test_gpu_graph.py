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


def _capture_and_compare(work, outputs, reset):
    """Eager run, then a captured graph of the same work replayed four times with
    eager work in between; every replay must reproduce the eager outputs bit for bit."""
    reset()
    work()
    torch.cuda.synchronize()
    want = [o.cpu().numpy().copy() for o in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        reset()
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work()
    for rep in range(4):
        reset()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert np.array_equal(o.cpu().numpy().view(np.uint32), w.view(np.uint32)), rep
        _ = torch.randn(1000, device="cuda").sum().item()


@pytest.mark.parametrize("kind", ["f32_tree65", "bf16_tree200", "chain300"])
def test_graph_replays_of_wider_paths(kind):
    """fp32 inputs (the coefficient + verify pair at 65 nodes), a 200-node tree and a
    300-token chunked chain with a final state, captured and replayed."""
    import workloads as W
    from gpu_support import to_dev
    G = require_gpu()
    rng = np.random.default_rng(7000 + len(kind))
    hk, hv, d_ = 2, 6, 128
    f32 = kind.startswith("f32")
    if kind == "chain300":
        n, B = 300, 1
        trees = None
    else:
        par = W.ddtree_tree(rng, 64 if kind == "f32_tree65" else 199, 8, 16)
        trees = [par, W.random_tree(rng, 9, 5)]
        B = len(trees)
        n = max(len(t) for t in trees)
    T = n * B if trees is None else sum(len(t) for t in trees)

    def vec(*shape):
        x = rng.standard_normal(shape)
        x /= np.linalg.norm(x, axis=-1, keepdims=True)
        x = x.astype(np.float32)
        return x if f32 else W.f32_to_bf16_bits(x)
    x = {"q": to_dev(vec(T, hk, d_)), "k": to_dev(vec(T, hk, d_)),
         "v": to_dev(rng.standard_normal((T, hv, d_)).astype(np.float32) if f32 else
                     W.f32_to_bf16_bits(rng.standard_normal((T, hv, d_)).astype(np.float32))),
         "a": to_dev(rng.uniform(0.5, 1.0, (T, hv)).astype(np.float32)),
         "b": to_dev(rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32))}
    S0 = to_dev((0.3 * rng.standard_normal((B, hv, d_, d_))).astype(np.float32))
    slots = to_dev(np.arange(B, dtype=np.int32))
    dims = G.make_dims(B, T, n, hk, hv, d_, B, G.GDN_F32 if f32 else G.GDN_BF16)
    ws = G.new_workspace(dims)
    out = torch.empty((T, hv, d_), device="cuda")
    if trees is None:
        cu = to_dev(np.array([0, n], np.int32))
        fl = to_dev(np.array([287], np.int32))
        fin = torch.empty((1, hv, d_, d_), device="cuda")

        def work():
            G.gdn_chain_verify(dims, cu, x["q"], x["k"], x["v"], x["a"], x["b"], S0, slots, out, fl, fin, ws)

        def reset():
            out.fill_(float("nan"))
            fin.fill_(float("nan"))
        outputs = [out, fin]
    else:
        parent = to_dev(np.concatenate(trees).astype(np.int32))
        cu = to_dev(W.cu_from_trees(trees).astype(np.int32))
        acc = to_dev(np.array([int(np.argmax(W.tree_depths(t))) for t in trees], np.int32))
        cache = S0.clone()

        def work():
            G.gdn_tree_plan(dims, parent, cu, slots, ws)
            G.gdn_tree_verify(dims, x["q"], x["k"], x["v"], x["a"], x["b"], cache, slots, out, ws)
            G.gdn_tree_persist(dims, x["k"], x["v"], x["a"], x["b"], acc, cache, slots, ws)

        def reset():
            cache.copy_(S0)
            out.fill_(float("nan"))
            ws.zero_()
        outputs = [out, cache]
    print("graph replay %s" % kind, flush=True)
    _capture_and_compare(work, outputs, reset)

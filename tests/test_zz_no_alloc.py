"""gdn_tree_verify_static (plan + verify with the library's static per-GPU
scratch instead of a caller workspace) against the existing entry points,
gdn_tree_plan + gdn_tree_verify, on two calls in a row, the second smaller:
the same outputs bit for bit, the same verdicts, and both within the oracle's
bar.  Dims whose plan would not fit the scratch are refused before any launch."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_support import TOL, require_gpu, slice_rel_err, to_dev

pytestmark = pytest.mark.gpu


def _case(rng, sizes, hk, hv, d_, bad_slot_seq=None):
    trees = [W.random_tree(rng, int(n), 16) for n in sizes]
    cu = W.cu_from_trees(trees).astype(np.int32)
    T = int(cu[-1])
    q = rng.standard_normal((T, hk, d_))
    k = rng.standard_normal((T, hk, d_))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    inp = {"q": W.f32_to_bf16_bits(q.astype(np.float32)), "k": W.f32_to_bf16_bits(k.astype(np.float32)),
           "v": W.f32_to_bf16_bits(rng.standard_normal((T, hv, d_)).astype(np.float32)),
           "a": rng.uniform(0.3, 1.0, (T, hv)).astype(np.float32), "b": rng.uniform(0.0, 1.0, (T, hv)).astype(np.float32)}
    B = len(sizes)
    num_slots = B + 2
    slots = rng.permutation(num_slots)[:B].astype(np.int32)
    if bad_slot_seq is not None:
        slots[bad_slot_seq] = num_slots + 5  # rejected by the plan
    cache = (0.3 * rng.standard_normal((num_slots, hv, d_, d_))).astype(np.float32)
    return trees, cu, inp, slots, cache


def _run_both(G, trees, cu, inp, slots, cache, hk, hv, d_):
    B, T = len(trees), int(cu[-1])
    max_nodes = max(len(t) for t in trees)
    dims = G.make_dims(B, T, max_nodes, hk, hv, d_, cache.shape[0], G.GDN_BF16)
    dev = {key: to_dev(val) for key, val in inp.items()}
    par_d, cu_d, slots_d, cache_d = (to_dev(x) for x in (np.concatenate(trees).astype(np.int32), cu, slots, cache))
    # the existing entry points, with a caller workspace
    ws = G.new_workspace(dims)
    ref = torch.full((T, hv, d_), float("nan"), device="cuda")
    G.gdn_tree_plan(dims, par_d, cu_d, slots_d, ws)
    G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d, slots_d, ref, ws)
    ref_status = G.read_metadata(dims, ws)["seq_status"].clone()
    # the allocation-free entry point
    out = torch.full((T, hv, d_), float("nan"), device="cuda")
    status = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    G.gdn_tree_verify_static(dims, par_d, cu_d, slots_d, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], cache_d,
                             out, status)
    torch.cuda.synchronize()
    assert np.array_equal(cache_d.cpu().numpy().view(np.uint32), cache.view(np.uint32))  # the cache is only read
    return out.cpu().numpy(), ref.cpu().numpy(), status.cpu().numpy(), ref_status.cpu().numpy()


@pytest.mark.parametrize("d_", [64, 128])
def test_static_verify_matches_workspace_verify_twice(d_):
    G = require_gpu()
    rng = np.random.default_rng(77 + d_)
    hk, hv = 4, 12
    # first call: 40 sequences of 1-90 nodes (the multi-block verify), one rejected;
    # second call, smaller: 6 sequences of up to 30 nodes (the single-block verify)
    for sizes, bad in ((rng.integers(1, 91, size=40), 7), (rng.integers(1, 31, size=6), None)):
        trees, cu, inp, slots, cache = _case(rng, sizes, hk, hv, d_, bad_slot_seq=bad)
        print("static verify: %d sequences, %d nodes, d=%d" % (len(sizes), int(cu[-1]), d_), flush=True)
        got, ref, status, ref_status = _run_both(G, trees, cu, inp, slots, cache, hk, hv, d_)
        assert np.array_equal(status, ref_status)
        assert (status != 0).sum() == (0 if bad is None else 1)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
        for s in range(len(sizes)):
            lo, hi = int(cu[s]), int(cu[s + 1])
            if status[s] != 0:
                assert np.isnan(got[lo:hi]).all()
                continue
            exp = oracle.tree(trees[s], inp["q"][lo:hi], inp["k"][lo:hi], inp["v"][lo:hi], inp["a"][lo:hi],
                              inp["b"][lo:hi], cache[slots[s]])
            assert slice_rel_err(got[lo:hi].transpose(1, 0, 2).reshape(hv, -1),
                                 exp.transpose(1, 0, 2).reshape(hv, -1)) <= TOL, s


def test_static_verify_refuses_dims_beyond_its_scratch():
    """A plan larger than the 32 MiB scratch: refused with GDN_ERR_WORKSPACE, nothing launched."""
    G = require_gpu()
    B, T, hv = 64, 64 * 200, 64  # about 4.1 kB of plan and coefficients per node and 64 heads
    dims = G.make_dims(B, T, 200, 16, hv, 128, B, G.GDN_BF16)
    assert G.workspace_bytes(dims) > 32 << 20
    z = lambda n, dt=torch.int32: torch.zeros(n, dtype=dt, device="cuda")  # noqa: E731
    out = torch.zeros((T, hv, 128), device="cuda")
    with pytest.raises(G.GdnError) as e:
        G.gdn_tree_verify_static(dims, z(T), z(B + 1), z(B), z(T * 16 * 128, torch.bfloat16).view(T, 16, 128),
                                 z(T * 16 * 128, torch.bfloat16).view(T, 16, 128),
                                 z(T * hv * 128, torch.bfloat16).view(T, hv, 128), z(T * hv, torch.float32),
                                 z(T * hv, torch.float32), torch.zeros((B, hv, 128, 128), device="cuda"), out)
    assert e.value.code == -4

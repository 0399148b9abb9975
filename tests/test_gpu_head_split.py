"""Head grouping of the matrix-core verify.  A workgroup takes all value heads
of its key head (GDN_VERIFY_HEADS=shared) or one value head (=split); the
automatic choice splits when one workgroup per value head all fit the device at
once.  Both groupings run the same arithmetic per head, so their outputs must
agree bit for bit: checked on the group kernel (23-node trees, 16-token chains)
and on the node-block kernel (65-node trees), at batch sizes on both sides of
the automatic switch.  Oracle parity of each grouping is covered by the head
group and sweep tests."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads as W
from gpu_support import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _inputs(name, num_seqs):
    cfg = W.get_config(name)
    if num_seqs is not None:
        cfg = dataclasses.replace(cfg, num_seqs=num_seqs, num_slots=num_seqs)
    trees = W.make_trees(cfg)
    cu = W.cu_from_trees(trees)
    inp = W.make_layer_inputs(cfg, 0, trees)
    rng = np.random.default_rng(5)
    cache = (0.05 * rng.standard_normal((cfg.num_slots, cfg.num_v_heads, cfg.head_dim, cfg.head_dim))).astype(np.float32)
    return cfg, trees, cu, inp, cache


def _verify(G, monkeypatch, heads, cfg, trees, cu, inp, cache, chain):
    monkeypatch.setenv("GDN_VERIFY_HEADS", heads)
    T = int(cu[-1])
    dims = G.make_dims(cfg.num_seqs, T, cfg.max_nodes, cfg.num_k_heads, cfg.num_v_heads, cfg.head_dim,
                       cfg.num_slots, G.GDN_BF16)
    ws = G.new_workspace(dims)
    dev = {k: to_dev(v) for k, v in inp.items()}
    slots = to_dev(W.make_slots(cfg).astype(np.int32))
    out = torch.full((T, cfg.num_v_heads, cfg.head_dim), float("nan"), device="cuda")
    if chain:
        G.gdn_chain_verify(dims, to_dev(cu.astype(np.int32)), dev["q"], dev["k"], dev["v"], dev["a"], dev["b"],
                           to_dev(cache), slots, out, None, None, ws)
    else:
        G.gdn_tree_plan(dims, to_dev(np.concatenate(trees).astype(np.int32)), to_dev(cu.astype(np.int32)), slots, ws)
        G.gdn_tree_verify(dims, dev["q"], dev["k"], dev["v"], dev["a"], dev["b"], to_dev(cache), slots, out, ws)
    rc, bad, code = G.gdn_tree_status(ws)
    assert rc == 0, (rc, bad, code)
    return out.cpu().numpy()


@pytest.mark.parametrize("name,num_seqs,chain", [
    ("ddtree22", None, False),   # one 23-node tree: group kernel, split by default
    ("batched", 4, False),
    ("batched", None, False),    # 32 sequences: shared by default
    ("chain", None, True),       # one 16-token chain through gdn_chain_verify
    ("stress", 2, False),        # 65-node trees: node-block kernel, split by default
    ("stress", 8, False),        # shared by default
])
def test_split_equals_shared(name, num_seqs, chain, monkeypatch):
    G = require_gpu()
    cfg, trees, cu, inp, cache = _inputs(name, num_seqs)
    print("head split", name, "B", cfg.num_seqs, "chain" if chain else "tree", flush=True)
    shared = _verify(G, monkeypatch, "shared", cfg, trees, cu, inp, cache, chain)
    split = _verify(G, monkeypatch, "split", cfg, trees, cu, inp, cache, chain)
    auto = _verify(G, monkeypatch, "auto", cfg, trees, cu, inp, cache, chain)
    assert np.isfinite(shared).all()
    assert np.array_equal(shared.view(np.uint32), split.view(np.uint32))
    assert np.array_equal(shared.view(np.uint32), auto.view(np.uint32))

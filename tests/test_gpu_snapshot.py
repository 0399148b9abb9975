"""Prefix-cache snapshots on the GPU (gdn_state_copy): bit-exact against the
oracle's copy, and a warm start (restore from the pool) continues bit for bit
like a cold one (prefill recomputed) through plan, verify and persist."""
import numpy as np
import pytest
import torch

import oracle.snapshot as snap
import workloads as W
from gpu_support import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _bits(rng, shape):
    """Arbitrary fp32 bit patterns, NaN payloads and -0 included."""
    return rng.integers(0, 2**32, size=shape, dtype=np.uint64).astype(np.uint32).view(np.float32)


@pytest.mark.parametrize("hv,d", [(48, 128), (2, 16), (3, 64)])
def test_copy_is_bit_exact(hv, d):
    G = require_gpu()
    rng = np.random.default_rng(hv * d)
    src = _bits(rng, (40, hv, d, d))
    dst = _bits(rng, (33, hv, d, d))
    src_slot = rng.permutation(40)[:32].astype(np.int32)
    dst_slot = rng.permutation(33)[:32].astype(np.int32)
    src_slot[3], dst_slot[7] = 40, -2          # skipped entries
    exp = snap.copy_slots(src, src_slot, dst, dst_slot)
    s_d, d_d = to_dev(src), to_dev(dst)
    G.gdn_state_copy(s_d, to_dev(src_slot), d_d, to_dev(dst_slot))
    torch.cuda.synchronize()
    assert np.array_equal(d_d.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    assert np.array_equal(s_d.cpu().numpy().view(np.uint32), src.view(np.uint32))


def test_copy_within_one_cache():
    G = require_gpu()
    rng = np.random.default_rng(3)
    cache = _bits(rng, (8, 4, 32, 32))
    src_slot = np.array([0, 1, 2], dtype=np.int32)
    dst_slot = np.array([5, 7, 6], dtype=np.int32)
    exp = snap.copy_slots(cache, src_slot, cache, dst_slot)
    c = to_dev(cache)
    G.gdn_state_copy(c, to_dev(src_slot), c, to_dev(dst_slot))
    torch.cuda.synchronize()
    assert np.array_equal(c.cpu().numpy().view(np.uint32), exp.view(np.uint32))


@pytest.mark.parametrize("name", ["ddtree22", "batched"])
def test_warm_start_equals_cold_start(name):
    G = require_gpu()
    cfg = W.get_config(name)
    trees = W.make_trees(cfg)
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    B, hv, hk, d, P = cfg.num_seqs, cfg.num_v_heads, cfg.num_k_heads, cfg.head_dim, cfg.prefill_steps
    inp = {k: to_dev(v) for k, v in W.make_layer_inputs(cfg, 0, trees).items()}
    pre = W.make_prefill(cfg, 0)
    slots = to_dev(W.make_slots(cfg))
    acc = to_dev(W.make_accepts(cfg, trees))
    parent = to_dev(np.concatenate(trees).astype(np.int32))
    cu_d = to_dev(cu.astype(np.int32))
    dims = G.make_dims(B, T, cfg.max_nodes, hk, hv, d, cfg.num_slots, G.GDN_BF16)
    # cold: the committed states come straight from prefill
    pre_dims = G.make_dims(B, B * P, P, hk, hv, d, cfg.num_slots, G.GDN_BF16)
    pre_cu = torch.arange(0, (B + 1) * P, P, dtype=torch.int32, device="cuda")
    zero = torch.zeros((cfg.num_slots, hv, d, d), device="cuda")
    fin = torch.empty((B, hv, d, d), device="cuda")
    G.gdn_chain_verify(pre_dims, pre_cu, None, to_dev(pre["k"].reshape(-1, hk, d)), to_dev(pre["v"].reshape(-1, hv, d)),
                       to_dev(pre["a"].reshape(-1, hv)), to_dev(pre["b"].reshape(-1, hv)), zero,
                       torch.arange(B, dtype=torch.int32, device="cuda"), None,
                       torch.full((B,), P, dtype=torch.int32, device="cuda"), fin)
    cold = torch.zeros((cfg.num_slots, hv, d, d), device="cuda")
    cold[slots.long()] = fin
    # warm: save the prefilled states into a prefix pool, wipe, restore into the same slots
    pool = torch.full((B + 3, hv, d, d), float("nan"), device="cuda")
    pool_slots = torch.arange(3, B + 3, dtype=torch.int32, device="cuda")
    G.gdn_state_copy(cold, slots, pool, pool_slots)
    warm = cold.clone()
    warm[slots.long()] = -5.0
    G.gdn_state_copy(pool, pool_slots, warm, slots)
    outs = []
    for cache in (cold, warm):
        ws = G.new_workspace(dims)
        out = torch.empty((T, hv, d), device="cuda")
        G.gdn_tree_plan(dims, parent, cu_d, slots, ws)
        G.gdn_tree_verify(dims, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], cache, slots, out, ws)
        G.gdn_tree_persist(dims, inp["k"], inp["v"], inp["a"], inp["b"], acc, cache, slots, ws)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), cache.cpu().numpy()))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))

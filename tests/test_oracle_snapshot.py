"""Prefix-cache snapshot oracle (CPU): a save followed by a restore gives the
state back bit for bit, and a warm start (restore, then verify) equals a cold
one (prefill, then verify) bit for bit in the fp64 oracle."""
import numpy as np

import oracle
import oracle.snapshot as snap
import workloads as W


def test_save_restore_roundtrip_and_skips():
    rng = np.random.default_rng(0)
    cache = rng.standard_normal((6, 2, 4, 4)).astype(np.float32)
    pool = np.zeros((3, 2, 4, 4), dtype=np.float32)
    pool = snap.copy_slots(cache, [4, 1, 9], pool, [0, 2, 1])      # source 9 is out of range
    assert np.array_equal(pool[0].view(np.uint32), cache[4].view(np.uint32))
    assert np.array_equal(pool[2].view(np.uint32), cache[1].view(np.uint32))
    assert not pool[1].any()
    junk = rng.standard_normal(cache.shape).astype(np.float32)
    back = snap.copy_slots(pool, [0, 2, 0], junk, [4, 1, -1])      # destination -1 is skipped
    assert np.array_equal(back[4].view(np.uint32), cache[4].view(np.uint32))
    assert np.array_equal(back[1].view(np.uint32), cache[1].view(np.uint32))
    for s in (0, 2, 3, 5):
        assert np.array_equal(back[s].view(np.uint32), junk[s].view(np.uint32))


def test_cold_equals_warm_in_the_oracle():
    cfg = W.get_config("tiny")
    trees = W.make_trees(cfg)
    inp = W.make_layer_inputs(cfg, 0, trees)
    pre = W.make_prefill(cfg, 0)
    cold = oracle.initial_states(pre, cfg.num_v_heads, cfg.head_dim)      # prefill from zero
    pool = snap.copy_slots(cold, [0], np.zeros((2,) + cold.shape[1:], np.float32), [1])
    warm = snap.copy_slots(pool, [1], np.full(cold.shape, 7.0, np.float32), [0])
    cu = W.cu_from_trees(trees)
    o_cold = oracle.verify_batch(trees, cu, inp, cold)
    o_warm = oracle.verify_batch(trees, cu, inp, warm)
    assert np.array_equal(o_cold.view(np.uint64), o_warm.view(np.uint64))

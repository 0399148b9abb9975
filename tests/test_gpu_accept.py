"""Greedy acceptance on the GPU (gdn_tree_accept) against the oracle
(oracle/accept.py): every row's argmax, the accepted node, the accept length
and the next token must match exactly."""
import numpy as np
import pytest
import torch

import oracle.accept as acc_oracle
import oracle.plan as oplan
import workloads as W
from workloads import draft
from gpu_support import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _run(G, trees, tok, logits, max_nodes=None, slots=None, num_slots=None, logits_dev=None, cu=None,
         parent=None):
    """plan + accept; returns (accepted, accept_len, next_token, target) as numpy."""
    B = len(trees) if cu is None else len(cu) - 1
    cu = W.cu_from_trees(trees) if cu is None else np.asarray(cu, dtype=np.int32)
    parent = np.concatenate(trees).astype(np.int32) if parent is None else np.asarray(parent, dtype=np.int32)
    T = int(cu[-1])
    slots = np.arange(B, dtype=np.int32) if slots is None else slots
    num_slots = max(B, 1) if num_slots is None else num_slots
    max_nodes = max([len(t) for t in trees] + [1]) if max_nodes is None else max_nodes
    dims = G.make_dims(B, T, max_nodes, 1, 1, 16, num_slots, G.GDN_F32)
    ws = G.new_workspace(dims)
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu), to_dev(slots.astype(np.int32)), ws)
    outs = [torch.full((B,), 12345, dtype=torch.int32, device="cuda") for _ in range(3)]
    tgt = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    lg = to_dev(logits) if logits_dev is None else logits_dev
    G.gdn_tree_accept(dims, lg, to_dev(np.asarray(tok, dtype=np.int32)), outs[0], outs[1], outs[2], ws,
                      target_token=tgt)
    torch.cuda.synchronize()
    return tuple(o.cpu().numpy() for o in outs) + (tgt.cpu().numpy(),)


def _expect(trees, tok, logits, slots=None, num_slots=None, max_nodes=None, cu=None, parent=None):
    cu = W.cu_from_trees(trees) if cu is None else np.asarray(cu)
    parent = np.concatenate(trees) if parent is None else np.asarray(parent)
    B = len(cu) - 1
    slots = np.arange(B) if slots is None else slots
    num_slots = max(B, 1) if num_slots is None else num_slots
    max_nodes = max([len(t) for t in trees] + [1]) if max_nodes is None else max_nodes
    status = oplan.validate(parent, cu, slots, num_slots, max_nodes, 16)
    return acc_oracle.accept(parent, cu, tok, logits, status)


def _check(got, exp):
    names = ("accepted_node", "accept_len", "next_token", "target_token")
    for g, e, nm in zip(got, exp, names):
        assert np.array_equal(g, e), "%s differs at %s: got %s, expected %s" % (
            nm, np.flatnonzero(g != e)[:8], g[g != e][:8], e[g != e][:8])


def _random_parent(rng, n, width, max_depth=16):
    par, dep, nk = [-1], [1], [0]
    for i in range(1, n):
        cand = [j for j in range(i) if nk[j] < width and dep[j] < max_depth]
        p = cand[int(rng.integers(len(cand)))]
        par.append(p)
        dep.append(dep[p] + 1)
        nk[p] += 1
        nk.append(0)
    return np.array(par, dtype=np.int32)


def test_accept_batched_full_vocab():
    """32 budget-22 trees, V = 248,320: every row's argmax and every sequence's
    outcome exact."""
    G = require_gpu()
    cfg = W.get_config("batched")
    trees = W.make_trees(cfg)
    tok = draft.make_draft_tokens(cfg, trees)
    logits = draft.make_verify_logits(cfg, trees, tok)
    got = _run(G, trees, tok, logits)
    exp = _expect(trees, tok, logits)
    _check(got, exp)
    assert exp[1].max() > 2  # the recipe accepts deep paths too


@pytest.mark.parametrize("vocab", [1, 3, 4, 97, 4096, 8193, 65537, 100003])
def test_accept_vocab_sizes(vocab):
    """Scalar and 16-byte paths, one to eight row slices, ragged slice tails."""
    G = require_gpu()
    cfg = W.get_config("ddtree22")
    rng = np.random.default_rng(vocab)
    trees = [_random_parent(rng, int(rng.integers(1, 30)), 4) for _ in range(5)]
    tok = draft.make_draft_tokens(cfg, trees, vocab)
    logits = draft.make_verify_logits(cfg, trees, tok, vocab)
    _check(_run(G, trees, tok, logits), _expect(trees, tok, logits))


@pytest.mark.parametrize("vocab", [5, 20000, 70001])
def test_accept_special_values(vocab):
    """NaNs, ties between slices, +0/-0, all -inf rows, +inf, ties with +inf."""
    G = require_gpu()
    rng = np.random.default_rng(7 + vocab)
    n = 12
    trees = [np.arange(-1, n - 1, dtype=np.int32)]
    logits = rng.standard_normal((n, vocab)).astype(np.float32)
    last = vocab - 1
    mid = vocab // 2
    logits[0, :] = -np.inf                                   # all -inf: index 0
    logits[1, last] = np.nan                                 # NaN at the very end wins
    logits[1, 0] = 1e30
    logits[2, [mid, last]] = np.nan                          # first NaN
    logits[3, [1, mid, last]] = 50.0                         # ties across slices: first
    logits[4, :] = 0.0
    logits[4, 0] = -0.0                                      # -0 equals +0: index 0
    logits[5, :] = -0.0
    logits[5, last] = 0.0
    logits[6, [min(2, last), last]] = np.inf                 # +inf tie
    logits[7, :] = -np.inf
    logits[7, last] = -3e38                                  # only finite entry at the end
    logits[8, mid] = np.inf
    logits[8, last] = np.nan                                 # NaN beats +inf
    logits[9, :] = np.float32(1.5)                           # constant row
    logits[10, [0, mid]] = [np.nan, 2.0]
    logits[11, mid:] = 9.0
    tok = np.zeros(n, dtype=np.int32)
    exp = _expect(trees, tok, logits)
    for k in range(1, n):  # make the chain accept as far as row k-1's argmax allows
        tok[k] = exp[3][k - 1]
    exp = _expect(trees, tok, logits)
    _check(_run(G, trees, tok, logits), exp)


def test_accept_unaligned_logits():
    """A logits base that is 4- but not 16-byte aligned takes the scalar loads."""
    G = require_gpu()
    cfg = W.get_config("ddtree22")
    vocab = 40000
    trees = W.make_trees(cfg)
    tok = draft.make_draft_tokens(cfg, trees, vocab)
    logits = draft.make_verify_logits(cfg, trees, tok, vocab)
    buf = torch.empty(logits.size + 1, dtype=torch.float32, device="cuda")
    view = buf[1:].view(logits.shape)
    view.copy_(torch.from_numpy(logits))
    assert view.data_ptr() % 16 != 0
    _check(_run(G, trees, tok, logits, logits_dev=view), _expect(trees, tok, logits))


def test_accept_rejected_empty_forest_and_foreign_tokens():
    G = require_gpu()
    rng = np.random.default_rng(3)
    vocab = 300
    trees = [
        np.array([-1, 0, 0, 1], dtype=np.int32),
        np.zeros(0, dtype=np.int32),                     # empty
        np.array([-1, 0, 5, 1], dtype=np.int32),          # bad parent id
        np.array([2, -1, 1, -1, 3], dtype=np.int32),      # forest, roots 1 and 3
        np.array([-1, 0, 1, 2], dtype=np.int32),
    ]
    parent = np.concatenate(trees)
    T = len(parent)
    logits = rng.standard_normal((T, vocab)).astype(np.float32)
    cu = W.cu_from_trees(trees)
    tok = rng.integers(0, vocab, T).astype(np.int32)
    # sequence 0 accepts 0 -> 1 -> 3; the forest accepts 1 -> 2 -> 0
    want = {(0, 1): (0,), (0, 3): (1,), (3, 2): (1,), (3, 0): (2,)}
    for (s, c), (p,) in want.items():
        tok[cu[s] + c] = int(np.argmax(logits[cu[s] + p]))
    # sequence 4: out-of-range tokens never match, even where the argmax is planted there
    tok[cu[4] + 1] = -1
    tok[cu[4] + 2] = vocab
    exp = _expect(trees, tok, logits)
    assert list(exp[0]) == [3, -1, -1, 0, 0] and list(exp[1]) == [3, 0, 0, 3, 1]
    _check(_run(G, trees, tok, logits), exp)


def test_accept_large_trees_and_stress_shapes():
    """Trees of up to 256 nodes (four per lane) and the stress workload's 65-node trees."""
    G = require_gpu()
    rng = np.random.default_rng(5)
    vocab = 2048
    cfg = W.get_config("stress")
    trees = [_random_parent(rng, 256, 3), _random_parent(rng, 200, 8), _random_parent(rng, 65, 2)]
    trees += W.make_trees(cfg)[:8]
    tok = draft.make_draft_tokens(cfg, trees, vocab)
    logits = draft.make_verify_logits(cfg, trees, tok, vocab, match=(0.9, 0.05))
    exp = _expect(trees, tok, logits)
    _check(_run(G, trees, tok, logits, max_nodes=256), exp)
    assert exp[1].max() >= 6


def test_accept_feeds_persist():
    """The accepted node from the GPU drives gdn_tree_persist; the slot then holds
    the oracle's replay of the oracle's accepted path."""
    import oracle
    from gpu_support import host_case, device_case, slice_rel_err, TOL
    G = require_gpu()
    case = host_case("ddtree22")
    cfg = case["cfg"]
    vocab = 32000
    tok = draft.make_draft_tokens(cfg, case["trees"], vocab)
    logits = draft.make_verify_logits(cfg, case["trees"], tok, vocab, match=(0.95,))
    exp = _expect(case["trees"], tok, logits)
    d = device_case(G, case)
    G.gdn_tree_plan(d["dims"], d["parent"], d["cu"], d["slots"], d["ws"])
    acc, alen, nxt = (torch.empty(cfg.num_seqs, dtype=torch.int32, device="cuda") for _ in range(3))
    G.gdn_tree_accept(d["dims"], to_dev(logits), to_dev(tok), acc, alen, nxt, d["ws"])
    G.gdn_tree_persist(d["dims"], d["k"], d["v"], d["a"], d["b"], acc, d["cache"], d["slots"], d["ws"])
    torch.cuda.synchronize()
    assert acc.cpu().numpy()[0] == exp[0][0] and alen.cpu().numpy()[0] == exp[1][0]
    state, path = oracle.accept_state(case["trees"][0], int(exp[0][0]), case["inp"]["k"], case["inp"]["v"],
                                      case["inp"]["a"], case["inp"]["b"], case["S0"][0])
    assert len(path) == exp[1][0]
    got = d["cache"].cpu().numpy()[case["slots"][0]]
    assert slice_rel_err(got.reshape(cfg.num_v_heads, -1), state.reshape(cfg.num_v_heads, -1)) <= TOL


def test_hand_worked_example():
    """The acceptance example worked by hand (tests/golden) on the GPU: exactly the
    hand-derived targets, accepted nodes, lengths and next tokens."""
    import accept_pins
    G = require_gpu()
    ex, logits = accept_pins.golden_accept_example()
    cu = np.array(ex["cu_nodes"], np.int32)
    trees = [np.array(ex["parent"][cu[s]:cu[s + 1]], np.int32) for s in range(len(cu) - 1)]
    got = _run(G, trees, ex["draft_token"], logits)
    for g, key in zip(got, ("accepted_node", "accept_len", "next_token", "target")):
        assert np.array_equal(g, ex[key]), (key, g)

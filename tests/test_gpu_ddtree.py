"""Draft top-k (gdn_draft_topk) and the DDTree builder (gdn_ddtree_build) on the
GPU against the oracle (oracle/ddtree.py).

Candidate ids, tree parents, node tokens and cu_nodes must match exactly; log
p values within the tolerance derived here.  The log-softmax is x - (m + log S) with S a sum of
up to 2.5e5 exponentials accumulated in fp32 (each term within 2 ulp, a
pairwise-tree sum of relative error ~18 x 6e-8) and the final subtraction
rounded at ulp(|x|) ~ 1e-6 |x|: a few 1e-6 in absolute terms, bounded here by
2e-5 + 1e-6 |x|."""
import numpy as np
import pytest
import torch

import oracle.ddtree as dd
import workloads as W
from workloads import draft
from gpu_support import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _topk(G, x, width, dev_x=None):
    rows = x.shape[0]
    tok = torch.full((rows, width), -7, dtype=torch.int32, device="cuda")
    lp = torch.full((rows, width), 7.0, dtype=torch.float32, device="cuda")
    G.gdn_draft_topk(to_dev(x) if dev_x is None else dev_x, width, tok, lp)
    torch.cuda.synchronize()
    return tok.cpu().numpy(), lp.cpu().numpy()


def _check_topk(x, got_t, got_lp, width):
    et, elp = dd.draft_topk(x, width)
    assert np.array_equal(got_t, et), np.argwhere(got_t != et)[:5]
    same_nan = np.isnan(got_lp) == np.isnan(elp)
    assert same_nan.all()
    fin = np.isfinite(elp)
    assert (np.isinf(got_lp) == np.isinf(elp)).all() and (got_lp[np.isinf(elp)] == elp[np.isinf(elp)]).all()
    xv = np.take_along_axis(x.astype(np.float64), np.maximum(et, 0), axis=1)
    tol = 2e-5 + 1e-6 * np.abs(xv)
    with np.errstate(invalid="ignore"):
        err = np.abs(got_lp.astype(np.float64) - elp)
    assert (err[fin] <= tol[fin]).all(), err[fin].max()
    return float(err[fin].max()) if fin.any() else 0.0


@pytest.mark.parametrize("width", [4, 8, 16])
def test_topk_full_vocab(width):
    """480 rows (32 sequences x 15 drafted positions) over V = 248,320."""
    G = require_gpu()
    cfg = W.get_config("batched")
    x = draft.make_draft_logits(cfg, width=width).reshape(-1, draft.VOCAB)
    t, lp = _topk(G, x, width)
    err = _check_topk(x, t, lp, width)
    print("max |log p error| %.2e" % err)


@pytest.mark.parametrize("vocab", [1, 3, 5, 17, 4096, 10001, 65536])
@pytest.mark.parametrize("width", [1, 3, 8, 16])
def test_topk_sizes(vocab, width):
    G = require_gpu()
    rng = np.random.default_rng(vocab * 31 + width)
    x = rng.standard_normal((6, vocab)).astype(np.float32)
    x[1] = np.round(x[1])            # many exact ties
    x[2] = -np.abs(x[2]) * 0.0       # all zero, some -0
    _check_topk(x, *_topk(G, x, width), width)


def test_topk_special_rows():
    G = require_gpu()
    rng = np.random.default_rng(1)
    V = 20000
    x = rng.standard_normal((10, V)).astype(np.float32)
    x[0, [17, 9000, 19999]] = np.nan
    x[1, :] = -np.inf
    x[2, 5000] = np.inf
    x[3, :] = -np.inf
    x[3, [4, 19998]] = [1.0, 2.0]
    x[4, [3, 7, 12000]] = 30.0       # ties at the top
    x[5, :] = 88.0                   # large equal logits: exp stays finite after the shift
    x[6, 100] = -3e38
    x[7, :] = np.float32(-1e30)
    x[7, 6] = np.nan
    # every value one thread reads in the first block is NaN (16 of them: four 16-byte
    # loads, one per 1024- or 512-thread stride for the short or the long lists), and a
    # larger finite value elsewhere: the NaNs still lead
    for row, threads in ((8, 1024), (9, 512)):
        for u in range(4):
            for c in range(4):
                x[row, 4 * (u * threads + 5) + c] = np.nan
        x[row, 3] = 1e30
    for width in (1, 4, 16):
        _check_topk(x, *_topk(G, x, width), width)


def test_topk_unaligned_rows():
    G = require_gpu()
    rng = np.random.default_rng(4)
    V = 4000
    x = rng.standard_normal((5, V)).astype(np.float32)
    buf = torch.empty(x.size + 1, dtype=torch.float32, device="cuda")
    view = buf[1:].view(x.shape)
    view.copy_(torch.from_numpy(x))
    _check_topk(x, *_topk(G, x, 4, dev_x=view), 4)


def _build(G, roots, tokens, logp, budget, max_depth=16):
    B, L, Wd = tokens.shape
    n = G.ddtree_nodes(L, Wd, budget, max_depth)
    par = torch.full((B * n,), -9, dtype=torch.int32, device="cuda")
    tok = torch.full((B * n,), -9, dtype=torch.int32, device="cuda")
    cu = torch.full((B + 1,), -9, dtype=torch.int32, device="cuda")
    G.gdn_ddtree_build(None if roots is None else to_dev(roots), to_dev(tokens.astype(np.int32)),
                       to_dev(logp.astype(np.float32)), budget, par, tok, cu, max_depth=max_depth)
    torch.cuda.synchronize()
    return par.cpu().numpy(), tok.cpu().numpy(), cu.cpu().numpy()


def _levels(rng, B, L, Wd, ties):
    if ties:
        lp = -rng.choice([0.25, 0.5, 1.0, 1.5, 2.0], size=(B, L, Wd))
    else:
        z = rng.normal(0.0, 2.0, size=(B, L, Wd))
        lp = z - np.log(np.exp(z).sum(axis=2, keepdims=True))
    return (-np.sort(-lp, axis=2)).astype(np.float32)


@pytest.mark.parametrize("L,Wd,budget,max_depth", [
    (15, 4, 22, 16), (15, 8, 64, 16), (15, 4, 255, 16), (15, 1, 40, 16), (3, 2, 100, 16), (15, 4, 0, 16),
    (15, 16, 200, 16), (15, 3, 50, 6), (20, 2, 30, 16), (1, 5, 9, 16), (15, 4, 22, 1)])
@pytest.mark.parametrize("ties", [False, True])
def test_builder_exact(L, Wd, budget, max_depth, ties):
    G = require_gpu()
    rng = np.random.default_rng(L * 1000 + Wd * 10 + budget + ties)
    B = 9
    lp = _levels(rng, B, L, Wd, ties)
    tokens = rng.integers(0, 248320, size=(B, L, Wd)).astype(np.int32)
    roots = rng.integers(0, 248320, size=B).astype(np.int32)
    got = _build(G, roots, tokens, lp, budget, max_depth)
    exp = dd.build_batch(roots, tokens, lp, budget, max_depth)
    for g, e, name in zip(got, exp, ("parent", "node_token", "cu_nodes")):
        assert np.array_equal(g, e), (name, np.flatnonzero(g != e)[:8])


def test_builder_nan_and_inf_log_probs_and_no_roots():
    G = require_gpu()
    rng = np.random.default_rng(8)
    B, L, Wd = 4, 15, 4
    lp = _levels(rng, B, L, Wd, False)
    lp[0, 3, 1:] = np.nan
    lp[1, :, 2:] = -np.inf
    lp[2, 0, :] = -np.inf
    lp[3, 5, 0] = np.nan
    tokens = rng.integers(0, 1000, size=(B, L, Wd)).astype(np.int32)
    got = _build(G, None, tokens, lp, 40)
    exp = dd.build_batch(np.full(B, -1), tokens, lp, 40)
    for g, e in zip(got, exp):
        assert np.array_equal(g, e)


def test_pipeline_topk_build_plan_accept():
    """Draft logits -> top-k -> tree -> plan -> greedy acceptance, all on the GPU.
    Candidate ids are exact, so the chain pre-seed and every tree whose
    best-first choices the oracle makes with a score margin above the
    accumulated log-p tolerance must match the oracle's tree exactly; the
    other trees must still obey the limits and carry the GPU's candidates."""
    import oracle.accept as acc_oracle
    import oracle.plan as oplan
    G = require_gpu()
    cfg = W.get_config("batched")
    vocab = 50000
    Wd, budget, L = cfg.tree[2], cfg.tree[1], draft.DRAFT_LEVELS
    B = cfg.num_seqs
    x = draft.make_draft_logits(cfg, vocab)
    roots = draft.make_root_tokens(cfg, vocab)
    tk = torch.empty((B * L, Wd), dtype=torch.int32, device="cuda")
    lpd = torch.empty((B * L, Wd), dtype=torch.float32, device="cuda")
    G.gdn_draft_topk(to_dev(x.reshape(-1, vocab)), Wd, tk, lpd)
    n = G.ddtree_nodes(L, Wd, budget)
    par = torch.empty(B * n, dtype=torch.int32, device="cuda")
    ntok = torch.empty(B * n, dtype=torch.int32, device="cuda")
    cu = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    G.gdn_ddtree_build(to_dev(roots), tk.view(B, L, Wd), lpd.view(B, L, Wd), budget, par, ntok, cu)
    torch.cuda.synchronize()
    et, elp = dd.draft_topk(x.reshape(-1, vocab), Wd)
    assert np.array_equal(tk.cpu().numpy(), et)
    et, elp = et.reshape(B, L, Wd), elp.reshape(B, L, Wd)
    gp, gt = par.cpu().numpy().reshape(B, n), ntok.cpu().numpy().reshape(B, n)
    ep_all, et_all, exact_seqs = [], [], []
    for b in range(B):
        margins = []
        ep, etok, _ = dd.build_tree(int(roots[b]), et[b], elp[b], budget, margins=margins)
        ep_all.append(ep)
        et_all.append(etok)
        if min(margins, default=np.inf) > 2e-3:
            assert np.array_equal(gp[b], ep) and np.array_equal(gt[b], etok), b
            exact_seqs.append(b)
        else:  # a near-tie: only structure
            assert gp[b][0] == -1 and all(0 <= gp[b][i] < i for i in range(1, n))
            assert list(gp[b][1:L + 1]) == list(range(L))
    print("%d of %d trees compared id for id" % (len(exact_seqs), B))
    assert len(exact_seqs) >= B // 2
    assert np.array_equal(cu.cpu().numpy(), np.arange(B + 1) * n)
    # the built trees go straight into plan + acceptance; the verify logits and the
    # expected outcome come from the oracle's trees, compared where the trees agree
    dims = G.make_dims(B, B * n, n, 1, 1, 16, B, G.GDN_F32)
    ws = G.new_workspace(dims)
    G.gdn_tree_plan(dims, par, cu, torch.arange(B, dtype=torch.int32, device="cuda"), ws)
    e_tok = np.concatenate(et_all)
    vlog = draft.make_verify_logits(cfg, ep_all, e_tok, vocab)
    outs = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(3)]
    G.gdn_tree_accept(dims, to_dev(vlog), ntok, outs[0], outs[1], outs[2], ws)
    rc = G.gdn_tree_status(ws)
    assert rc[0] == 0
    cu_h = np.arange(B + 1) * n
    status = oplan.validate(np.concatenate(ep_all), cu_h, np.arange(B), B, n, 16)
    ea = acc_oracle.accept(np.concatenate(ep_all), cu_h, e_tok, vlog, status)
    for g, e in zip(outs, ea[:3]):
        g = g.cpu().numpy()
        assert np.array_equal(g[exact_seqs], e[exact_seqs])


def test_builder_no_sequences():
    G = require_gpu()
    cu = torch.full((1,), -9, dtype=torch.int32, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    G.gdn_ddtree_build(None, torch.empty((0, 15, 4), dtype=torch.int32, device="cuda"),
                       torch.empty((0, 15, 4), dtype=torch.float32, device="cuda"), 22, e, e, cu)
    torch.cuda.synchronize()
    assert cu.item() == 0


def test_builder_hand_worked_example():
    """The builder on the hand-worked example (tests/golden), twice in one batch:
    parents, node tokens and cu_nodes exactly as derived by hand."""
    import ddtree_pins
    G = require_gpu()
    ex = ddtree_pins.golden_ddtree_example()
    tokens = np.array([ex["tokens"]] * 2, np.int32)
    logp = np.array([ex["logp"]] * 2, np.float32)
    roots = np.array([ex["root_token"]] * 2, np.int32)
    par, tok, cu = _build(G, roots, tokens, logp, ex["budget"], ex["max_depth"])
    n = len(ex["parent"])
    assert list(cu) == [0, n, 2 * n]
    assert list(par) == ex["parent"] * 2 and list(tok) == ex["node_token"] * 2

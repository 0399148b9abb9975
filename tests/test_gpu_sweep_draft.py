"""Seeded sweeps of greedy acceptance, the DDTree builder and the draft top-k
against the oracle: random forests and relabelled trees of 1-96 nodes with tied
and NaN logits; builder levels, widths, budgets and depth caps with exactly tied
dyadic scores and impossible candidates; top-k over ragged vocabularies with
ties, NaN, +inf and all -inf rows.  Integer outputs bit for bit, log
probabilities within the top-k tests' bound."""
import numpy as np
import pytest
import torch

import oracle.accept as acc_oracle
import oracle.ddtree as dd
import oracle.plan as oplan
import workloads as W
from gpu_support import require_gpu, to_dev

pytestmark = pytest.mark.gpu
CASES = 8


@pytest.mark.parametrize("seed", range(CASES))
def test_accept_sweep(seed):
    G = require_gpu()
    rng = np.random.default_rng(5000 + seed)
    B = int(rng.integers(1, 9))
    V = int(rng.choice([1, 2, 7, 100, 4097, 20000]))
    trees = []
    for _ in range(B):
        n = int(rng.integers(1, 97))
        par = W.random_tree(rng, n, int(rng.integers(2, 17)) if n > 1 else 1)
        if rng.random() < 0.3:
            par = W.relabel(par, rng.permutation(n))
        trees.append(par.astype(np.int32))
    cu = W.cu_from_trees(trees)
    T = int(cu[-1])
    parent = np.concatenate(trees).astype(np.int32)
    logits = rng.standard_normal((T, V)).astype(np.float32)
    if rng.random() < 0.5:
        logits = np.round(logits).astype(np.float32)  # ties
    for r in np.flatnonzero(rng.random(T) < 0.05):
        logits[r, rng.integers(0, V)] = np.nan
    tok = rng.integers(-2, V + 2, size=T).astype(np.int32)
    tgt = acc_oracle.target_tokens(logits)
    for s, par in enumerate(trees):  # make matches likely
        lo = int(cu[s])
        for i, p in enumerate(par):
            if p >= 0 and rng.random() < 0.6:
                tok[lo + i] = tgt[lo + int(p)]
    print("accept sweep", seed, "B", B, "V", V, "nodes", [len(t) for t in trees], flush=True)
    dims = G.make_dims(B, T, max(len(t) for t in trees), 1, 1, 16, B, G.GDN_F32)
    ws = G.new_workspace(dims)
    G.gdn_tree_plan(dims, to_dev(parent), to_dev(cu.astype(np.int32)), to_dev(np.arange(B, dtype=np.int32)), ws)
    outs = [torch.full((B,), 777, dtype=torch.int32, device="cuda") for _ in range(3)]
    tg = torch.full((T,), -7, dtype=torch.int32, device="cuda")
    G.gdn_tree_accept(dims, to_dev(logits), to_dev(tok), outs[0], outs[1], outs[2], ws, target_token=tg)
    torch.cuda.synchronize()
    status = oplan.validate(parent, cu, np.arange(B), B, dims.max_nodes, 16)
    exp = acc_oracle.accept(parent, cu, tok, logits, status)
    for got, want in zip([o.cpu().numpy() for o in outs] + [tg.cpu().numpy()], exp):
        assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(CASES))
def test_builder_sweep(seed):
    G = require_gpu()
    rng = np.random.default_rng(7000 + seed)
    B = int(rng.integers(1, 6))
    L = int(rng.integers(1, 21))
    Wd = int(rng.integers(1, 17))
    budget = int(rng.integers(0, 256))
    md = int(rng.integers(1, 17))
    n = G.ddtree_nodes(L, Wd, budget, md)
    assert n == dd.tree_size(L, Wd, budget, md)
    if rng.random() < 0.5:  # exactly tied dyadic scores
        lp = -rng.choice([0.25, 0.5, 1.0, 1.5, 2.0], size=(B, L, Wd))
    else:
        z = rng.normal(0.0, 2.0, size=(B, L, Wd))
        lp = z - np.log(np.exp(z).sum(axis=2, keepdims=True))
    lp = (-np.sort(-lp, axis=2)).astype(np.float32)
    if rng.random() < 0.3:
        lp[0, int(rng.integers(0, L)), -1] = -np.inf
    tokens = rng.integers(0, 248320, size=(B, L, Wd)).astype(np.int32)
    roots = rng.integers(0, 248320, size=B).astype(np.int32)
    print("builder sweep", seed, "B", B, "levels", L, "width", Wd, "budget", budget, "depth cap", md, "nodes", n,
          flush=True)
    par = torch.full((B * n,), -9, dtype=torch.int32, device="cuda")
    nt = torch.full((B * n,), -9, dtype=torch.int32, device="cuda")
    cuo = torch.full((B + 1,), -9, dtype=torch.int32, device="cuda")
    G.gdn_ddtree_build(to_dev(roots), to_dev(tokens), to_dev(lp), budget, par, nt, cuo, max_depth=md)
    torch.cuda.synchronize()
    for got, want in zip((par.cpu().numpy(), nt.cpu().numpy(), cuo.cpu().numpy()),
                         dd.build_batch(roots, tokens, lp, budget, md)):
        assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(CASES))
def test_topk_sweep(seed):
    G = require_gpu()
    rng = np.random.default_rng(9000 + seed)
    rows = int(rng.integers(1, 20))
    V = int(rng.choice([1, 3, 16, 257, 4096, 9999, 70001]))
    Wd = int(rng.integers(1, 17))
    x = rng.standard_normal((rows, V)).astype(np.float32)
    if rng.random() < 0.5:
        x = np.round(x * 2).astype(np.float32)
    for r in range(rows):
        u = rng.random()
        if u < 0.05:
            x[r, rng.integers(0, V)] = np.nan
        elif u < 0.1:
            x[r, :] = -np.inf
        elif u < 0.15:
            x[r, rng.integers(0, V)] = np.inf
    print("top-k sweep", seed, "rows", rows, "vocab", V, "width", Wd, flush=True)
    tk = torch.full((rows, Wd), -7, dtype=torch.int32, device="cuda")
    lpo = torch.full((rows, Wd), 7.0, device="cuda")
    G.gdn_draft_topk(to_dev(x), Wd, tk, lpo)
    torch.cuda.synchronize()
    et, elp = dd.draft_topk(x, Wd)
    gt, gl = tk.cpu().numpy(), lpo.cpu().numpy()
    assert np.array_equal(gt, et)
    assert (np.isnan(gl) == np.isnan(elp)).all()
    assert (np.isinf(gl) == np.isinf(elp)).all() and (gl[np.isinf(elp)] == elp[np.isinf(elp)]).all()
    fin = np.isfinite(elp)
    xv = np.take_along_axis(x.astype(np.float64), np.maximum(et, 0), axis=1)
    with np.errstate(invalid="ignore"):
        err = np.abs(gl.astype(np.float64) - elp)
    assert (err[fin] <= (2e-5 + 1e-6 * np.abs(xv))[fin]).all()

"""Draft top-k / DDTree builder oracle: its pins, planted mistakes, and the
seeded draft-logits recipe (CPU only)."""
import importlib.util

import numpy as np
import pytest

import ddtree_pins
import oracle.ddtree as dd
import workloads as W
from workloads import draft

SRC = dd.__file__


@pytest.mark.parametrize("pin", ddtree_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(dd)


MUTANTS = {
    "no_chain_preseed": ("while len(parent) - 1 < budget and depth[cur] < depth_cap and W > 0:",
                         "while False:"),
    "rank_before_depth": ("heapq.heappush(heap, (-float(s), depth[par] + 1, r, par))",
                          "heapq.heappush(heap, (-float(s), r, depth[par] + 1, par))"),
    "larger_parent_first": ("heapq.heappush(heap, (-float(s), depth[par] + 1, r, par))",
                            "heapq.heappush(heap, (-float(s), depth[par] + 1, r, -par))"),
    "level_of_parent": ("        s = np.float32(score[par] + lp[depth[par] - 1, r])",
                        "        s = np.float32(score[par] + lp[max(depth[par] - 2, 0), r])"),
    "depth_limit_off_by_one": ("    depth_cap = min(L + 1, max_depth)\n", "    depth_cap = min(L + 2, max_depth + 1)\n"),
    "width_limit_off_by_one": ("if depth[par] >= depth_cap or nchild[par] >= W:", "if depth[par] >= depth_cap or nchild[par] > W:"),
    "topk_larger_id_first": ("order = np.lexsort((idx, -np.where(nan, 0.0, x), ~nan))",
                             "order = np.lexsort((-idx, -np.where(nan, 0.0, x), ~nan))"),
    "topk_nan_last": ("order = np.lexsort((idx, -np.where(nan, 0.0, x), ~nan))",
                      "order = np.lexsort((idx, -np.where(nan, 0.0, x), nan))"),
    "logp_without_normalizer": ("logp[r, :w] = x[order[:w]] - (m + np.log(np.exp(x - m).sum()))",
                                "logp[r, :w] = x[order[:w]] - m"),
    "token_of_rank_one": ("token.append(int(tokens[depth[par] - 1, r]))", "token.append(int(tokens[depth[par] - 1, 0]))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site not found: " + name
    path = tmp_path / ("dd_%s.py" % name)
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("dd_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    failed = []
    for pin in ddtree_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, "planted mistake %r passed every pin" % name


def test_draft_logits_recipe():
    cfg = W.get_config("batched")
    vocab = 5000
    x = draft.make_draft_logits(cfg, vocab)
    assert x.shape == (cfg.num_seqs, draft.DRAFT_LEVELS, vocab) and x.dtype == np.float32
    assert np.array_equal(x, draft.make_draft_logits(cfg, vocab))
    tok, lp = dd.draft_topk(x.reshape(-1, vocab), cfg.tree[2])
    # peaked like a drafter: the rank-1 candidate usually carries most of the mass
    assert np.median(np.exp(lp[:, 0])) > 0.3
    roots = draft.make_root_tokens(cfg, vocab)
    par, t, cu = dd.build_batch(roots, tok.reshape(cfg.num_seqs, draft.DRAFT_LEVELS, -1),
                                lp.reshape(cfg.num_seqs, draft.DRAFT_LEVELS, -1), cfg.tree[1])
    assert cu[-1] == cfg.num_seqs * (cfg.tree[1] + 1)

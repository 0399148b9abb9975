"""Greedy-acceptance oracle: its pins, planted mistakes, and the seeded draft
token / logits recipe (CPU only)."""
import importlib.util
import os

import numpy as np
import pytest

import accept_pins
import oracle.accept as acc_oracle
import workloads as W
from workloads import draft

SRC = acc_oracle.__file__


@pytest.mark.parametrize("pin", accept_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(acc_oracle)


MUTANTS = {
    "compare_at_child": ("want = int(target[cur])\n", "want = None\n"),
    "walk_uses_largest_child": ("cur = min(kids)", "cur = max(kids)"),
    "length_counts_drafts_only": ("    length = 1\n", "    length = 0\n"),
    "next_from_parent_row": ("nxt[s] = node, length, target[lo + node]", "nxt[s] = node, length, draft_token[lo + node]"),
    "argmax_last_tie": ("return np.argmax(logits, axis=1).astype(np.int32)",
                        "return (logits.shape[1] - 1 - np.argmax(logits[:, ::-1], axis=1)).astype(np.int32)"),
    "argmax_ignores_nan": ("return np.argmax(logits, axis=1).astype(np.int32)",
                           "return np.nanargmax(np.where(np.isnan(logits), -np.inf, logits), axis=1).astype(np.int32)"),
    "largest_root": ("cur = min(i for i in range(n) if parent[i] == -1)", "cur = max(i for i in range(n) if parent[i] == -1)"),
    "rejected_still_walked": ("if int(status[s]) != SEQ_OK or hi <= lo:", "if hi <= lo:"),
}


def _load_mutant(tmp_path, name):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation site not found: " + name
    text = src.replace(old, new)
    if name == "compare_at_child":  # compare each child with its own row
        text = text.replace("int(draft_token[c]) == want]", "int(draft_token[c]) == int(target[c])]")
    text = text.replace("from .plan import SEQ_OK", "SEQ_OK = 0")
    path = tmp_path / ("acc_%s.py" % name)
    path.write_text(text)
    spec = importlib.util.spec_from_file_location("acc_%s" % name, str(path))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    mod = _load_mutant(tmp_path, name)
    failed = []
    for pin in accept_pins.ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, TypeError, IndexError):
            failed.append(pin.__name__)
    assert failed, "planted mistake %r passed every pin" % name


def test_draft_recipe_siblings_distinct_and_seeded():
    cfg = W.get_config("batched")
    trees = W.make_trees(cfg)[:4]
    tok = draft.make_draft_tokens(cfg, trees)
    tok2 = draft.make_draft_tokens(cfg, trees)
    assert np.array_equal(tok, tok2)
    assert tok.min() >= 0 and tok.max() < draft.VOCAB
    lo = 0
    for par in trees:
        for u in range(len(par)):
            sib = [int(tok[lo + c]) for c in range(len(par)) if par[c] == u]
            assert len(sib) == len(set(sib))
        lo += len(par)


def test_logits_recipe_accepts_plausible_lengths():
    cfg = W.get_config("batched")
    trees = W.make_trees(cfg)[:8]
    vocab = 4096
    tok = draft.make_draft_tokens(cfg, trees, vocab)
    logits = draft.make_verify_logits(cfg, trees, tok, vocab)
    assert logits.dtype == np.float32 and logits.shape == (sum(len(t) for t in trees), vocab)
    cu = W.cu_from_trees(trees)
    acc, alen, nxt, tgt = acc_oracle.accept(np.concatenate(trees), cu, tok, logits, np.zeros(len(trees)))
    assert (alen >= 1).all() and alen.max() > 1
    for s in range(len(trees)):
        assert nxt[s] == tgt[cu[s] + acc[s]]


def test_hand_worked_example():
    """The acceptance example worked by hand (tests/golden): the oracle must give
    exactly the hand-derived targets, accepted nodes, lengths and next tokens."""
    import oracle.accept as acc
    ex, logits = accept_pins.golden_accept_example()
    got = acc.accept(np.array(ex["parent"], np.int32), np.array(ex["cu_nodes"]),
                     np.array(ex["draft_token"], np.int32), logits, np.zeros(len(ex["cu_nodes"]) - 1, np.int32))
    for g, key in zip(got, ("accepted_node", "accept_len", "next_token", "target")):
        assert np.array_equal(g, ex[key]), key

"""Planted mistakes: copies of the oracle's C source with one plausible
error each must fail at least one pin (CPU only).  This shows the pins are
strong enough to catch a dropped term, a wrong sign, a wrong index or a
transposed operand anywhere in the oracle."""
import os

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

MUTANTS = {
    "erase_sign": ("Si[j] - b * sk * k[j]", "Si[j] + b * sk * k[j]"),
    "no_decay": ("Oi[j] = a * (Si[j] - b * sk * k[j])", "Oi[j] = (Si[j] - b * sk * k[j])"),
    "decayed_write": ("+ b * v[i] * k[j];", "+ a * b * v[i] * k[j];"),
    "transposed_outer": ("+ b * v[i] * k[j];", "+ b * v[j] * k[i];"),
    "erase_without_b": ("Si[j] - b * sk * k[j]", "Si[j] - sk * k[j]"),
    "output_before_update": ("state_times(dv, dk, st + (size_t)i * ss, q", "state_times(dv, dk, par, q"),
    "parent_is_root": (": st + (size_t)parent[i] * ss;", ": S0 + (size_t)h * ss;"),
    "gqa_interleaved": ("        const int g = h / group;\n        double *st", "        const int g = h % hk;\n        double *st"),
    "persist_leaf_first": ("const int i = path[p];", "const int i = path[len - 1 - p];"),
    "persist_skips_root": ("for (int p = 0; p < len; ++p) {", "for (int p = 1; p < len; ++p) {"),
    "query_uses_key": ("q + ((size_t)i * hk + g) * dk,\n                        out", "k + ((size_t)i * hk + g) * dk,\n                        out"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new, 1)
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(mutated)
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmut_%s.so" % name)))
    failed = []
    with oracle.using_library(lib):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except (AssertionError, RuntimeError):
                failed.append(getattr(pin, "__name__", "brute"))
    assert failed, "planted mistake %r passed every pin" % name


def test_unmutated_copy_passes_all_pins(tmp_path):
    lib = oracle.compile_source(SRC, str(tmp_path / "libcopy.so"))
    with oracle.using_library(lib):
        for pin in pins.ALL_PINS:
            pin()


def _wrong_seq_state(trees, cu, inputs, S0_seq):
    """Mistake: every sequence starts from the first sequence's committed state."""
    return _orig_verify(trees, cu, inputs, [S0_seq[0]] * len(trees))


def _shifted_ranges(trees, cu, inputs, S0_seq):
    """Mistake: node ranges taken one sequence late (cu[s + 1] as the start)."""
    import numpy as np
    cu2 = np.concatenate([[0], cu[2:], [cu[-1]]])[: len(cu)]
    return _orig_verify(trees, cu2, inputs, S0_seq)


def _persist_skip_ignored(trees, cu, inputs, S0_seq, accepted):
    """Mistake: a skipped sequence (accepted -1) persists its last node."""
    import numpy as np
    acc = np.array([m if m >= 0 else len(t) - 1 for m, t in zip(accepted, trees)], np.int32)
    return _orig_persist(trees, cu, inputs, S0_seq, acc)


def _persist_wrong_state(trees, cu, inputs, S0_seq, accepted):
    """Mistake: persist replays from the last sequence's committed state."""
    return _orig_persist(trees, cu, inputs, [S0_seq[-1]] * len(trees), accepted)


_orig_verify = oracle.verify_batch
_orig_persist = oracle.persist_batch
WRAPPER_MUTANTS = {
    "verify_wrong_seq_state": ("verify_batch", _wrong_seq_state),
    "verify_shifted_ranges": ("verify_batch", _shifted_ranges),
    "persist_skip_ignored": ("persist_batch", _persist_skip_ignored),
    "persist_wrong_state": ("persist_batch", _persist_wrong_state),
}


@pytest.mark.parametrize("name", sorted(WRAPPER_MUTANTS))
def test_batch_wrapper_mutant_fails_its_pin(name, monkeypatch):
    """Plausible mistakes in the batch wrappers (the per-sequence slicing, state
    selection and skip handling) each fail pin_batch_wrappers."""
    attr, fn = WRAPPER_MUTANTS[name]
    monkeypatch.setattr(oracle, attr, fn)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pins.pin_batch_wrappers()

"""The C-ABI library loads and exports every entry point include/gdn_tree.h
declares; pure host-side calls behave as documented (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn_tree.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    import gated_deltanet_tree_amd as G
    if not os.path.exists(G.LIB_PATH):
        from gated_deltanet_tree_amd import build
        build.build()
    return G.load_library()


def test_header_declares_expected_entry_points():
    import gated_deltanet_tree_amd as G
    assert _declared() == sorted(G.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_host_only_calls(lib):
    import gated_deltanet_tree_amd as G
    dims = G.make_dims(32, 736, 23, 16, 48, 128, 32, G.GDN_BF16)
    n = G.workspace_bytes(dims)
    assert n > 0 and n % 256 == 0
    bad = G.make_dims(1, 4, 8, 2, 3, 128, 1, G.GDN_BF16)
    assert G.workspace_bytes(bad) == 0
    assert G.strerror(0) == "ok"
    assert "workspace" in G.strerror(-4)
    # argument errors are reported before anything touches the device
    assert lib.gdn_tree_plan(None, None, None, None, None, 0, None) == -1
    assert lib.gdn_tree_plan(ctypes.byref(dims), None, None, None, None, 0, None) == -1
    rc = lib.gdn_tree_verify(ctypes.byref(bad), None, None, None, None, None, None, None, None,
                             ctypes.c_void_p(1), 1 << 20, None)
    assert rc == -2
    assert lib.gdn_tree_status(None, 0, None, None, None) == -1


def test_accept_host_checks(lib):
    import gated_deltanet_tree_amd as G
    dims = G.make_dims(2, 10, 8, 1, 1, 16, 2, G.GDN_F32)
    one = ctypes.c_void_p(16)
    n = G.workspace_bytes(dims)
    assert lib.gdn_tree_accept(None, one, 10, one, one, one, one, None, one, n, None) == -1
    assert lib.gdn_tree_accept(ctypes.byref(dims), one, 0, one, one, one, one, None, one, n, None) == -2
    assert lib.gdn_tree_accept(ctypes.byref(dims), None, 10, one, one, one, one, None, one, n, None) == -1
    assert lib.gdn_tree_accept(ctypes.byref(dims), one, 10, one, None, one, one, None, one, n, None) == -1
    assert lib.gdn_tree_accept(ctypes.byref(dims), one, 10, one, one, one, one, None, None, n, None) == -1
    assert lib.gdn_tree_accept(ctypes.byref(dims), one, 10, one, one, one, one, None, one, n - 1, None) == -4


def test_draft_and_builder_host_checks(lib):
    one = ctypes.c_void_p(16)
    assert lib.gdn_draft_topk(4, 100, 0, one, one, one, None) == -2
    assert lib.gdn_draft_topk(4, 100, 17, one, one, one, None) == -2
    assert lib.gdn_draft_topk(4, 0, 4, one, one, one, None) == -2
    assert lib.gdn_draft_topk(4, 100, 4, None, one, one, None) == -1
    assert lib.gdn_draft_topk(0, 100, 4, None, None, None, None) == 0
    import oracle.ddtree as dd
    for args in [(15, 4, 22, 16), (15, 8, 64, 16), (3, 2, 100, 16), (15, 1, 40, 16), (5, 3, 0, 16), (15, 4, 22, 6)]:
        assert lib.gdn_ddtree_nodes(*args) == dd.tree_size(*args), args
    assert lib.gdn_ddtree_nodes(0, 4, 22, 16) == 0 and lib.gdn_ddtree_nodes(15, 17, 22, 16) == 0
    assert lib.gdn_ddtree_nodes(15, 4, 22, 17) == 0
    assert lib.gdn_ddtree_build(2, 15, 4, 300, 16, None, one, one, one, one, one, None) == -2
    assert lib.gdn_ddtree_build(2, 15, 4, 22, 16, None, None, one, one, one, one, None) == -1


def test_state_copy_host_checks(lib):
    one = ctypes.c_void_p(16)
    assert lib.gdn_state_copy(48, 128, one, 4, one, one, 4, one, 0, None) == 0
    assert lib.gdn_state_copy(0, 128, one, 4, one, one, 4, one, 2, None) == -2
    assert lib.gdn_state_copy(48, 126, one, 4, one, one, 4, one, 2, None) == -2
    assert lib.gdn_state_copy(48, 128, one, 4, one, one, 4, one, -1, None) == -2
    assert lib.gdn_state_copy(48, 128, None, 4, one, one, 4, one, 2, None) == -1
    assert lib.gdn_state_copy(48, 128, ctypes.c_void_p(20), 4, one, one, 4, one, 2, None) == -2


def test_missing_library_fails_loudly(tmp_path):
    """With no built library every entry point raises: there is no fallback path."""
    import gated_deltanet_tree_amd as G
    saved = G._lib
    G._lib = None
    try:
        with pytest.raises(ImportError, match="missing"):
            G.load_library(str(tmp_path / "libgdn_tree.so"))
    finally:
        G._lib = saved


def test_package_never_imports_the_oracle():
    """The product package holds no reference to the CPU oracle."""
    pkg = os.path.join(ROOT, "gated_deltanet_tree_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def test_persist_verify_host_checks(lib):
    """gdn_tree_persist_verify's argument errors are reported before anything is
    enqueued: the two steps' dims must agree in batch, heads, head dim, slots and
    dtype; required pointers; both workspaces large enough and apart."""
    import gated_deltanet_tree_amd as G
    one = ctypes.c_void_p(16)
    prev = G.make_dims(4, 60, 23, 2, 4, 64, 6, G.GDN_BF16)
    nxt = G.make_dims(4, 50, 20, 2, 4, 64, 6, G.GDN_BF16)   # node counts may differ
    n_p, n_n = G.workspace_bytes(prev), G.workspace_bytes(nxt)
    far = ctypes.c_void_p(1 << 40)

    def call(dp, dn, ws_p=one, nb_p=n_p, ws_n=far, nb_n=n_n, acc=one, out=one):
        return lib.gdn_tree_persist_verify(ctypes.byref(dp) if dp is not None else None, one, one, one, one, acc,
                                           ws_p, nb_p, ctypes.byref(dn) if dn is not None else None, one, one, one,
                                           one, one, one, one, out, ws_n, nb_n, None)

    assert call(None, nxt) == -1
    assert call(prev, None) == -1
    for field, value in [("num_seqs", 5), ("num_k_heads", 1), ("num_v_heads", 8), ("head_dim", 128),
                         ("num_slots", 7), ("qkv_dtype", G.GDN_F32)]:
        other = G.make_dims(4, 50, 20, 2, 4, 64, 6, G.GDN_BF16)
        setattr(other, field, value)
        if field == "num_seqs":
            other.num_slots = 6
        assert call(prev, other) == -2, field
    assert call(prev, nxt, ws_p=None) == -1
    assert call(prev, nxt, ws_n=None) == -1
    assert call(prev, nxt, acc=None) == -1
    assert call(prev, nxt, out=None) == -1
    assert call(prev, nxt, nb_p=n_p - 1) == -4
    assert call(prev, nxt, nb_n=n_n - 1) == -4
    assert call(prev, nxt, ws_n=one) == -4                            # one workspace for both steps
    assert call(prev, nxt, ws_n=ctypes.c_void_p(16 + n_p - 256)) == -4  # step t+1's starts inside step t's
    assert call(prev, nxt, ws_p=ctypes.c_void_p((1 << 40) + n_n - 256)) == -4
    empty = G.make_dims(0, 0, 1, 2, 4, 64, 0, G.GDN_BF16)
    n_e = G.workspace_bytes(empty)
    assert call(empty, empty, nb_p=n_e, nb_n=n_e) == 0  # nothing to do: returns before any launch

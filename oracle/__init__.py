"""fp64 CPU oracle for Gated DeltaNet tree verification and persistence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library (``gated_deltanet_tree_amd``) and never imports it.

Contents
  gdn_oracle.c  fp64 loops: sequential recurrence, tree verify (every node's
                state kept, nodes visited by increasing depth), accepted-path
                replay.  Built with gcc by ``build()``.
  plan.py       per-sequence verdicts and traversal metadata (pure Python).
  literal.py    the rule as an explicit matrix product, for tiny pins.

Inputs are numpy arrays in the library's layouts; bf16 values are passed as
uint16 bit patterns and widened exactly.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

from . import plan  # noqa: F401
from .plan import validate, plan_tree, stack_bound  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc, plain -O2: no fast-math, no FMA contraction."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-shared", "-fPIC", "-std=c11", "-Wall", "-o", tmp, src])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into oracle/libgdn_oracle.so."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        compile_source(_SRC, _LIB)
    return _LIB


def _declare(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int32)
    i = ctypes.c_int
    lib.oracle_chain.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_tree.argtypes = [i, ip, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp]
    lib.oracle_accept_state.argtypes = [i, ip, i, i, i, i, i, dp, dp, dp, dp, dp, dp, ip]
    lib.oracle_num_threads.argtypes = []
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_set_threads.restype = None
    for f in (lib.oracle_chain, lib.oracle_tree, lib.oracle_accept_state, lib.oracle_num_threads):
        f.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        build(force=False)
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


class using_library:
    """Context manager that points the wrappers at another build of
    gdn_oracle.c (used by the tests that plant mistakes in a copy)."""

    def __init__(self, path: str):
        self.path = path

    def __enter__(self):
        global _lib
        self.saved = _load()
        _lib = None
        lib = ctypes.CDLL(self.path)
        _lib = _declare(lib)
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_threads(n: int) -> None:
    """Threads the oracle's loops use from now on; 0 restores the default."""
    _load().oracle_set_threads(int(n))


def widen(x) -> np.ndarray:
    """Exact fp64 value of an input array (uint16 = bf16 bit patterns)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    return np.ascontiguousarray(x, dtype=np.float64)


def _dp(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _ip(x):
    return None if x is None else x.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def chain(k, v, a, b, S0, q=None):
    """Sequential recurrence over L tokens of one sequence.
    k [L,hk,d], v [L,hv,d], a/b [L,hv], S0 [hv,dv,dk], q [L,hk,d] or None.
    Returns (out [L,hv,dv] or None, final state [hv,dv,dk]) in fp64."""
    k, v, a, b, S0 = widen(k), widen(v), widen(a), widen(b), widen(S0)
    L, hk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    qq = None if q is None else widen(q)
    out = None if q is None else np.zeros((L, hv, dv))
    fin = np.zeros((hv, dv, dk))
    rc = _load().oracle_chain(L, hk, hv, dk, dv, _dp(qq), _dp(k), _dp(v), _dp(a), _dp(b), _dp(S0),
                              _dp(out), _dp(fin))
    if rc != 0:
        raise RuntimeError("oracle_chain failed: %d" % rc)
    return out, fin


def tree(parent, q, k, v, a, b, S0, return_states: bool = False):
    """Tree verify of one sequence.  Returns out [n,hv,dv] (and node states
    [n,hv,dv,dk] if asked) in fp64."""
    par = np.ascontiguousarray(parent, dtype=np.int32)
    q, k, v, a, b, S0 = widen(q), widen(k), widen(v), widen(a), widen(b), widen(S0)
    n = len(par)
    hk, dk = k.shape[1], k.shape[2]
    hv, dv = v.shape[1], v.shape[2]
    out = np.zeros((n, hv, dv))
    st = np.zeros((n, hv, dv, dk)) if return_states else None
    rc = _load().oracle_tree(n, _ip(par), hk, hv, dk, dv, _dp(q), _dp(k), _dp(v), _dp(a), _dp(b),
                             _dp(S0), _dp(out), _dp(st))
    if rc != 0:
        raise RuntimeError("oracle_tree failed: %d" % rc)
    return (out, st) if return_states else out


def accept_state(parent, m, k, v, a, b, S0):
    """Persist of one sequence: (new state [hv,dv,dk] fp64, path root-first)."""
    par = np.ascontiguousarray(parent, dtype=np.int32)
    k, v, a, b, S0 = widen(k), widen(v), widen(a), widen(b), widen(S0)
    n = len(par)
    hk, dk = k.shape[1], k.shape[2]
    hv, dv = v.shape[1], v.shape[2]
    out = np.zeros((hv, dv, dk))
    path = np.zeros(max(n, 1), dtype=np.int32)
    rc = _load().oracle_accept_state(n, _ip(par), int(m), hk, hv, dk, dv, _dp(k), _dp(v), _dp(a), _dp(b),
                                     _dp(S0), _dp(out), _ip(path))
    if rc < 0:
        raise RuntimeError("oracle_accept_state failed: %d" % rc)
    return out, path[:rc].copy()


def initial_states(prefill: dict, hv: int, d: int) -> np.ndarray:
    """Committed states built by the sequential recurrence from a zero state
    over each sequence's prefill tokens, rounded to fp32 (RNE).
    prefill: k [S,P,hk,d], v [S,P,hv,d], a/b [S,P,hv].  Returns [S,hv,d,d] f32."""
    nseq = prefill["a"].shape[0]
    out = np.empty((nseq, hv, d, d), dtype=np.float32)
    zero = np.zeros((hv, d, d))
    for s in range(nseq):
        _, fin = chain(prefill["k"][s], prefill["v"][s], prefill["a"][s], prefill["b"][s], zero)
        out[s] = fin.astype(np.float32)
    return out


def verify_batch(trees, cu, inputs, S0_seq):
    """Tree verify over all sequences.  S0_seq [B,hv,dv,dk] (committed state of
    each sequence).  Returns out [T,hv,dv] fp64."""
    T = int(cu[-1])
    hv, dv = inputs["v"].shape[1], inputs["v"].shape[2]
    out = np.zeros((T, hv, dv))
    for s, par in enumerate(trees):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if hi == lo:
            continue
        out[lo:hi] = tree(par, inputs["q"][lo:hi], inputs["k"][lo:hi], inputs["v"][lo:hi],
                          inputs["a"][lo:hi], inputs["b"][lo:hi], S0_seq[s])
    return out


def persist_batch(trees, cu, inputs, S0_seq, accepted):
    """Accepted-path states per sequence: list of (state fp64 or None, path)."""
    res = []
    for s, par in enumerate(trees):
        lo, hi = int(cu[s]), int(cu[s + 1])
        m = int(accepted[s])
        if m < 0 or hi == lo:
            res.append((None, np.zeros(0, dtype=np.int32)))
            continue
        res.append(accept_state(par, m, inputs["k"][lo:hi], inputs["v"][lo:hi], inputs["a"][lo:hi],
                                inputs["b"][lo:hi], S0_seq[s]))
    return res

"""Gated DeltaNet tree verify + accepted-path persist for MI355X (gfx950).

A thin ctypes binding over ``libgdn_tree.so`` (C ABI in ``include/gdn_tree.h``).
Every step of the path runs in the library's HIP kernels; this module only
checks tensors and passes their device pointers and the current HIP stream.
torch is used for device memory and streams, nothing else.

Typical decode step (all on one stream)::

    dims = make_dims(...)
    ws = torch.empty(workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    gdn_tree_plan(dims, parent, cu_nodes, slot_idx, ws)
    for layer in layers:
        gdn_tree_verify(dims, q, k, v, a, b, cache[layer], slot_idx, out, ws)
    gdn_tree_accept(dims, logits, draft_token, accepted, accept_len, next_token, ws)
    for layer in layers:
        gdn_tree_persist(dims, k, v, a, b, accepted, cache[layer], slot_idx, ws)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_tree.so")

GDN_MAX_DEPTH = 16
GDN_MAX_NODES = 256
GDN_MAX_CHAIN = 65536
GDN_MAX_DRAFT_WIDTH = 16
GDN_BF16, GDN_F32 = 0, 1

SEQ_STATUS = {0: "OK", 1: "BAD_NODES", 2: "BAD_SLOT", 3: "DUP_SLOT", 4: "BAD_PARENT",
              5: "CYCLE_OR_DEPTH", 6: "BAD_ACCEPT", 7: "NOT_PERSISTED"}

EXPORTS = ["gdn_workspace_bytes", "gdn_tree_plan", "gdn_tree_verify", "gdn_tree_persist",
           "gdn_chain_verify", "gdn_tree_accept", "gdn_draft_topk", "gdn_ddtree_nodes", "gdn_ddtree_build",
           "gdn_state_copy", "gdn_tree_verify_store", "gdn_tree_persist_copy", "gdn_tree_read_metadata",
           "gdn_tree_status", "gdn_strerror", "gdn_tree_verify_static", "gdn_probe_stream",
           "gdn_tree_persist_verify"]


class GdnError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, strerror(code), code))
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "num_seqs", "total_nodes", "max_nodes", "max_depth", "num_k_heads", "num_v_heads",
        "head_dim", "num_slots", "qkv_dtype")]

    def __repr__(self):
        return "Dims(%s)" % ", ".join("%s=%d" % (f, getattr(self, f)) for f, _ in self._fields_)


def make_dims(num_seqs, total_nodes, max_nodes, num_k_heads, num_v_heads, head_dim, num_slots,
              qkv_dtype=GDN_BF16, max_depth=GDN_MAX_DEPTH) -> Dims:
    return Dims(int(num_seqs), int(total_nodes), int(max_nodes), int(max_depth), int(num_k_heads),
                int(num_v_heads), int(head_dim), int(num_slots), int(qkv_dtype))


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libgdn_tree.so; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libgdn_tree.so is missing at %s; build it with "
                          "`python -m gated_deltanet_tree_amd.build`" % path)
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    dp = ctypes.POINTER(Dims)
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.gdn_workspace_bytes.argtypes = [dp]
    lib.gdn_workspace_bytes.restype = sz
    lib.gdn_tree_plan.argtypes = [dp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_verify.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_persist.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_persist_verify.argtypes = [dp, vp, vp, vp, vp, vp, vp, sz, dp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                            sz, vp]
    lib.gdn_tree_verify_static.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_probe_stream.argtypes = [ctypes.c_int32, vp, vp, sz, sz, vp]
    lib.gdn_chain_verify.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_accept.argtypes = [dp, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, sz, vp]
    i32c = ctypes.c_int32
    lib.gdn_draft_topk.argtypes = [i32c, i32c, i32c, vp, vp, vp, vp]
    lib.gdn_ddtree_nodes.argtypes = [i32c, i32c, i32c, i32c]
    lib.gdn_ddtree_nodes.restype = i32c
    lib.gdn_ddtree_build.argtypes = [i32c, i32c, i32c, i32c, i32c, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_state_copy.argtypes = [i32c, i32c, vp, i32c, vp, vp, i32c, vp, i32c, vp]
    lib.gdn_tree_verify_store.argtypes = [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_persist_copy.argtypes = [dp, vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_tree_read_metadata.argtypes = [dp, vp, sz, vp, vp, vp, vp, vp, vp, vp]
    lib.gdn_tree_status.argtypes = [vp, sz, vp, ip, ip]
    lib.gdn_strerror.argtypes = [i32]
    lib.gdn_strerror.restype = ctypes.c_char_p
    for f in ("gdn_tree_plan", "gdn_tree_verify", "gdn_tree_persist", "gdn_chain_verify",
              "gdn_tree_accept", "gdn_draft_topk", "gdn_ddtree_build", "gdn_state_copy", "gdn_tree_verify_store",
              "gdn_tree_persist_copy", "gdn_tree_read_metadata", "gdn_tree_status", "gdn_tree_verify_static",
              "gdn_probe_stream"):
        getattr(lib, f).restype = i32
    _lib = lib
    return lib


def strerror(code: int) -> str:
    return load_library().gdn_strerror(int(code)).decode()


# ---------------------------------------------------------------- checks
def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t, name, dtype=None, numel=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if numel is not None and t.numel() != numel:
        raise ValueError("%s has %d elements, expected %d" % (name, t.numel(), numel))
    return ctypes.c_void_p(t.data_ptr())


def _qkv_dtype(dims):
    return torch.bfloat16 if dims.qkv_dtype == GDN_BF16 else torch.float32


def _check(code, where):
    if code != 0:
        raise GdnError(code, where)


def workspace_bytes(dims: Dims) -> int:
    return int(load_library().gdn_workspace_bytes(ctypes.byref(dims)))


def new_workspace(dims: Dims, device="cuda") -> torch.Tensor:
    n = workspace_bytes(dims)
    if n == 0:
        raise ValueError("invalid dims %r" % dims)
    return torch.empty(n, dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def gdn_tree_plan(dims, parent, cu_nodes, slot_idx, ws, stream=None):
    T, B = dims.total_nodes, dims.num_seqs
    _check(load_library().gdn_tree_plan(
        ctypes.byref(dims), _ptr(parent, "parent", torch.int32, T), _ptr(cu_nodes, "cu_nodes", torch.int32, B + 1),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
        "gdn_tree_plan")


def gdn_tree_verify(dims, q, k, v, a, b, state_cache, slot_idx, out, ws, stream=None):
    T, B, Hk, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dt = _qkv_dtype(dims)
    _check(load_library().gdn_tree_verify(
        ctypes.byref(dims), _ptr(q, "q", dt, T * Hk * D), _ptr(k, "k", dt, T * Hk * D),
        _ptr(v, "v", dt, T * Hv * D), _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(out, "out", torch.float32, T * Hv * D),
        _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "gdn_tree_verify")


def gdn_tree_verify_static(dims, parent, cu_nodes, slot_idx, q, k, v, a, b, state_cache, out, seq_status=None,
                           stream=None):
    """Plan + verify with no workspace: the plan's metadata lives in the library's
    static per-GPU scratch.  seq_status (int32 [B]) receives the verdicts if given."""
    T, B, Hk, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dt = _qkv_dtype(dims)
    _check(load_library().gdn_tree_verify_static(
        ctypes.byref(dims), _ptr(parent, "parent", torch.int32, T), _ptr(cu_nodes, "cu_nodes", torch.int32, B + 1),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(q, "q", dt, T * Hk * D), _ptr(k, "k", dt, T * Hk * D),
        _ptr(v, "v", dt, T * Hv * D), _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(out, "out", torch.float32, T * Hv * D), _ptr(seq_status, "seq_status", torch.int32, B, allow_none=True),
        _stream(stream)), "gdn_tree_verify_static")


def gdn_probe_stream(mode, src, dst, stream=None):
    """Diagnostic streaming pass: mode "read" reads all of src (partial sums into
    dst), mode "copy" copies src into dst."""
    m = {"read": 0, "copy": 1}[mode]
    nbytes = src.numel() * src.element_size()
    _check(load_library().gdn_probe_stream(m, _ptr(src, "src"), _ptr(dst, "dst"), nbytes,
                                           dst.numel() * dst.element_size(), _stream(stream)), "gdn_probe_stream")


def gdn_tree_persist(dims, k, v, a, b, accepted_node, state_cache, slot_idx, ws, stream=None):
    T, B, Hk, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dt = _qkv_dtype(dims)
    _check(load_library().gdn_tree_persist(
        ctypes.byref(dims), _ptr(k, "k", dt, T * Hk * D), _ptr(v, "v", dt, T * Hv * D),
        _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(accepted_node, "accepted_node", torch.int32, B),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
        "gdn_tree_persist")


def gdn_tree_persist_verify(prev_dims, prev_k, prev_v, prev_a, prev_b, accepted_node, prev_ws, dims, q, k, v, a, b,
                            state_cache, slot_idx, out, ws, stream=None):
    """gdn_tree_persist of the previous step (prev_* and its workspace) followed by
    gdn_tree_verify of the next (dims, inputs, outputs, workspace) in one pass over the
    state cache."""
    Tp, T, B = prev_dims.total_nodes, dims.total_nodes, dims.num_seqs
    Hk, Hv, D = dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dtp, dt = _qkv_dtype(prev_dims), _qkv_dtype(dims)
    _check(load_library().gdn_tree_persist_verify(
        ctypes.byref(prev_dims), _ptr(prev_k, "prev_k", dtp, Tp * prev_dims.num_k_heads * prev_dims.head_dim),
        _ptr(prev_v, "prev_v", dtp, Tp * prev_dims.num_v_heads * prev_dims.head_dim),
        _ptr(prev_a, "prev_a", torch.float32, Tp * prev_dims.num_v_heads),
        _ptr(prev_b, "prev_b", torch.float32, Tp * prev_dims.num_v_heads),
        _ptr(accepted_node, "accepted_node", torch.int32, B), _ptr(prev_ws, "prev_ws", torch.uint8),
        prev_ws.numel(), ctypes.byref(dims), _ptr(q, "q", dt, T * Hk * D), _ptr(k, "k", dt, T * Hk * D),
        _ptr(v, "v", dt, T * Hv * D), _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(out, "out", torch.float32, T * Hv * D),
        _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "gdn_tree_persist_verify")


def gdn_tree_verify_store(dims, q, k, v, a, b, state_cache, slot_idx, out, node_states, ws, stream=None):
    """gdn_tree_verify plus every node's state in fp16 (node_states: torch.float16 [T, H_v, D, D])."""
    T, B, Hk, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dt = _qkv_dtype(dims)
    _check(load_library().gdn_tree_verify_store(
        ctypes.byref(dims), _ptr(q, "q", dt, T * Hk * D), _ptr(k, "k", dt, T * Hk * D),
        _ptr(v, "v", dt, T * Hv * D), _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(out, "out", torch.float32, T * Hv * D),
        _ptr(node_states, "node_states", torch.float16, T * Hv * D * D),
        _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "gdn_tree_verify_store")


def gdn_tree_persist_copy(dims, accepted_node, node_states, state_cache, slot_idx, ws, stream=None):
    """Commit by copy: the accepted node's stored fp16 state into each sequence's slot."""
    T, B, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_v_heads, dims.head_dim
    _check(load_library().gdn_tree_persist_copy(
        ctypes.byref(dims), _ptr(accepted_node, "accepted_node", torch.int32, B),
        _ptr(node_states, "node_states", torch.float16, T * Hv * D * D),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)),
        "gdn_tree_persist_copy")


def gdn_chain_verify(dims, cu_nodes, q, k, v, a, b, state_cache, slot_idx, out=None, final_len=None,
                     final_state=None, ws=None, stream=None):
    T, B, Hk, Hv, D = dims.total_nodes, dims.num_seqs, dims.num_k_heads, dims.num_v_heads, dims.head_dim
    dt = _qkv_dtype(dims)
    _check(load_library().gdn_chain_verify(
        ctypes.byref(dims), _ptr(cu_nodes, "cu_nodes", torch.int32, B + 1),
        _ptr(q, "q", dt, T * Hk * D, allow_none=True), _ptr(k, "k", dt, T * Hk * D), _ptr(v, "v", dt, T * Hv * D),
        _ptr(a, "a", torch.float32, T * Hv), _ptr(b, "b", torch.float32, T * Hv),
        _ptr(state_cache, "state_cache", torch.float32, dims.num_slots * Hv * D * D),
        _ptr(slot_idx, "slot_idx", torch.int32, B), _ptr(out, "out", torch.float32, T * Hv * D, allow_none=True),
        _ptr(final_len, "final_len", torch.int32, B, allow_none=True),
        _ptr(final_state, "final_state", torch.float32, B * Hv * D * D, allow_none=True),
        _ptr(ws, "ws", torch.uint8, allow_none=True), 0 if ws is None else ws.numel(), _stream(stream)),
        "gdn_chain_verify")


def gdn_tree_accept(dims, logits, draft_token, accepted_node, accept_len, next_token, ws, target_token=None,
                    stream=None):
    """Greedy acceptance: logits fp32 [T][vocab]; writes accepted_node, accept_len,
    next_token (int32 [B]) and, if given, target_token (int32 [T])."""
    T, B = dims.total_nodes, dims.num_seqs
    if logits is None or logits.dim() != 2 or logits.shape[0] != T:
        raise ValueError("logits must be a [T, vocab] tensor")
    vocab = int(logits.shape[1])
    _check(load_library().gdn_tree_accept(
        ctypes.byref(dims), _ptr(logits, "logits", torch.float32, T * vocab), vocab,
        _ptr(draft_token, "draft_token", torch.int32, T), _ptr(accepted_node, "accepted_node", torch.int32, B),
        _ptr(accept_len, "accept_len", torch.int32, B), _ptr(next_token, "next_token", torch.int32, B),
        _ptr(target_token, "target_token", torch.int32, T, allow_none=True),
        _ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream)), "gdn_tree_accept")


def gdn_draft_topk(logits, width, tokens, logp, stream=None):
    """logits fp32 [rows, vocab] -> tokens int32 [rows, width], logp fp32 [rows, width]."""
    if logits is None or logits.dim() != 2:
        raise ValueError("logits must be a [rows, vocab] tensor")
    rows, vocab = int(logits.shape[0]), int(logits.shape[1])
    _check(load_library().gdn_draft_topk(
        rows, vocab, int(width), _ptr(logits, "logits", torch.float32, rows * vocab),
        _ptr(tokens, "tokens", torch.int32, rows * width), _ptr(logp, "logp", torch.float32, rows * width),
        _stream(stream)), "gdn_draft_topk")


def ddtree_nodes(levels, width, budget, max_depth=GDN_MAX_DEPTH) -> int:
    """Nodes of every tree gdn_ddtree_build grows (0 for invalid arguments)."""
    return int(load_library().gdn_ddtree_nodes(int(levels), int(width), int(budget), int(max_depth)))


def gdn_ddtree_build(root_token, tokens, logp, budget, parent, node_token, cu_nodes, max_depth=GDN_MAX_DEPTH,
                     stream=None):
    """tokens int32 / logp fp32 [B, levels, width] -> parent, node_token int32 [B*N], cu_nodes [B+1]."""
    if tokens is None or tokens.dim() != 3:
        raise ValueError("tokens must be a [B, levels, width] tensor")
    B, L, Wd = (int(x) for x in tokens.shape)
    n = ddtree_nodes(L, Wd, budget, max_depth)
    _check(load_library().gdn_ddtree_build(
        B, L, Wd, int(budget), int(max_depth), _ptr(root_token, "root_token", torch.int32, B, allow_none=True),
        _ptr(tokens, "tokens", torch.int32, B * L * Wd), _ptr(logp, "logp", torch.float32, B * L * Wd),
        _ptr(parent, "parent", torch.int32, B * n), _ptr(node_token, "node_token", torch.int32, B * n),
        _ptr(cu_nodes, "cu_nodes", torch.int32, B + 1), _stream(stream)), "gdn_ddtree_build")


def gdn_state_copy(src_cache, src_slot, dst_cache, dst_slot, stream=None):
    """Prefix-cache snapshot: dst_cache[dst_slot[i]] = src_cache[src_slot[i]] (whole slots,
    caches fp32 [slots, H_v, D, D])."""
    if src_cache.dim() != 4 or dst_cache.dim() != 4 or src_cache.shape[1:] != dst_cache.shape[1:]:
        raise ValueError("caches must be [slots, H_v, D, D] tensors of the same slot shape")
    hv, d = int(src_cache.shape[1]), int(src_cache.shape[2])
    n = int(src_slot.numel())
    _check(load_library().gdn_state_copy(
        hv, d, _ptr(src_cache, "src_cache", torch.float32), int(src_cache.shape[0]),
        _ptr(src_slot, "src_slot", torch.int32, n), _ptr(dst_cache, "dst_cache", torch.float32),
        int(dst_cache.shape[0]), _ptr(dst_slot, "dst_slot", torch.int32, n), n, _stream(stream)), "gdn_state_copy")


def gdn_tree_read_metadata(dims, ws, depth=None, order=None, action=None, path=None, path_len=None,
                           seq_status=None, stream=None):
    T, B = dims.total_nodes, dims.num_seqs
    _check(load_library().gdn_tree_read_metadata(
        ctypes.byref(dims), _ptr(ws, "ws", torch.uint8), ws.numel(),
        _ptr(depth, "depth", torch.int32, T, True), _ptr(order, "order", torch.int32, T, True),
        _ptr(action, "action", torch.int32, T, True), _ptr(path, "path", torch.int32, B * GDN_MAX_DEPTH, True),
        _ptr(path_len, "path_len", torch.int32, B, True), _ptr(seq_status, "seq_status", torch.int32, B, True),
        _stream(stream)), "gdn_tree_read_metadata")


def gdn_tree_status(ws, stream=None):
    """Synchronizes the stream; returns (status, first_bad_seq, first_bad_code)."""
    seq = ctypes.c_int32(-1)
    code = ctypes.c_int32(0)
    rc = load_library().gdn_tree_status(_ptr(ws, "ws", torch.uint8), ws.numel(), _stream(stream),
                                        ctypes.byref(seq), ctypes.byref(code))
    return int(rc), int(seq.value), int(code.value)


def read_metadata(dims, ws, stream=None) -> dict:
    """Convenience: all metadata as fresh device tensors."""
    T, B = dims.total_nodes, dims.num_seqs
    dev = ws.device
    md = {
        "depth": torch.empty(T, dtype=torch.int32, device=dev),
        "order": torch.empty(T, dtype=torch.int32, device=dev),
        "action": torch.empty(T, dtype=torch.int32, device=dev),
        "path": torch.empty(B * GDN_MAX_DEPTH, dtype=torch.int32, device=dev),
        "path_len": torch.empty(B, dtype=torch.int32, device=dev),
        "seq_status": torch.empty(B, dtype=torch.int32, device=dev),
    }
    gdn_tree_read_metadata(dims, ws, stream=stream, **md)
    md["path"] = md["path"].view(B, GDN_MAX_DEPTH)
    return md

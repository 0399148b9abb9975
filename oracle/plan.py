"""Tree validation and traversal metadata, written out plainly in Python.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The draft tree arrives in parent-pointer form (local node ids, -1 marks a
root), as DDTree's ``build_ddtree`` produces it on the GreenGames page (section
"From autoregressive to DDTree").  Depth counts the nodes on the root-to-node
path, root = 1; depth is bounded by the drafting block of 16 tokens (section
"Prefill": the draft block size).

Per-sequence verdict codes (first failing check wins):
  0 OK
  1 BAD_NODES       node range [cu[b], cu[b+1]) not inside [0, T] or longer than max_nodes
  2 BAD_SLOT        slot_idx[b] outside [0, num_slots)              (non-empty sequences)
  3 DUP_SLOT        slot shared with another non-empty sequence      (all sharers flagged)
  4 BAD_PARENT      parent id outside {-1} U [0, n) or equal to the node itself
  5 CYCLE_OR_DEPTH  a node's ancestor walk does not reach a root within max_depth nodes
  6 BAD_ACCEPT      accepted node outside {-1} U [0, n)              (persist only)

Traversal (used by the recurrent verify): children of a node -- and the roots
of a forest -- are ordered by (subtree size, id) ascending, so the largest
subtree comes last; ``order`` is the depth-first preorder under that ordering.
Per visited position the action word holds
  bits 0-1  how the parent's state is obtained: 0 continue (it is the state
            just produced), 1 copy the stack top, 2 pop the stack top,
            3 reload the committed state (roots)
  bit 2     push the node's state (the node has >= 2 children)
  bit 3     leaf (no state update needed afterwards).
"""
from __future__ import annotations

import numpy as np

SEQ_OK, SEQ_BAD_NODES, SEQ_BAD_SLOT, SEQ_DUP_SLOT = 0, 1, 2, 3
SEQ_BAD_PARENT, SEQ_CYCLE_OR_DEPTH, SEQ_BAD_ACCEPT = 4, 5, 6

ACT_CONTINUE, ACT_TOP, ACT_POP, ACT_INIT = 0, 1, 2, 3
ACT_PUSH, ACT_LEAF = 4, 8

MAX_PATH = 16


def validate(parent, cu_nodes, slot_idx, num_slots: int, max_nodes: int, max_depth: int) -> np.ndarray:
    parent = np.asarray(parent, dtype=np.int64)
    cu = np.asarray(cu_nodes, dtype=np.int64)
    slots = np.asarray(slot_idx, dtype=np.int64)
    total = len(parent)
    nseq = len(cu) - 1
    status = np.zeros(nseq, dtype=np.int32)
    active = np.zeros(nseq, dtype=bool)
    for s in range(nseq):
        lo, hi = int(cu[s]), int(cu[s + 1])
        if not (0 <= lo <= hi <= total) or hi - lo > max_nodes:
            status[s] = SEQ_BAD_NODES
            continue
        active[s] = hi > lo
    for s in range(nseq):
        if active[s] and not (0 <= slots[s] < num_slots):
            status[s] = SEQ_BAD_SLOT
    for s in range(nseq):
        if not active[s] or status[s]:
            continue
        for o in range(nseq):
            if o != s and active[o] and 0 <= slots[o] < num_slots and slots[o] == slots[s]:
                status[s] = SEQ_DUP_SLOT
                break
    for s in range(nseq):
        if not active[s] or status[s]:
            continue
        lo, hi = int(cu[s]), int(cu[s + 1])
        n = hi - lo
        par = parent[lo:hi]
        if any(not (p == -1 or 0 <= p < n) or p == i for i, p in enumerate(par)):
            status[s] = SEQ_BAD_PARENT
            continue
        for i in range(n):
            j, steps = i, 0
            while j != -1 and steps < max_depth:
                steps += 1
                j = int(par[j])
            if j != -1:
                status[s] = SEQ_CYCLE_OR_DEPTH
                break
    return status


def plan_tree(par) -> dict:
    """Traversal metadata of one valid tree (local ids)."""
    par = [int(p) for p in par]
    n = len(par)
    depth = [0] * n
    for i in range(n):
        d, j = 0, i
        while j != -1:
            d += 1
            j = par[j]
        depth[i] = d
    size = [1] * n  # every node counts itself and adds itself to each ancestor
    for i in range(n):
        j = par[i]
        while j != -1:
            size[j] += 1
            j = par[j]
    children = [[] for _ in range(n)]
    roots = []
    for i in range(n):
        (roots if par[i] == -1 else children[par[i]]).append(i)
    key = lambda c: (size[c], c)  # noqa: E731
    roots.sort(key=key)
    for c in children:
        c.sort(key=key)

    order = []
    todo = list(reversed(roots))
    while todo:
        x = todo.pop()
        order.append(x)
        todo.extend(reversed(children[x]))

    action = []
    stack_len, max_stack = 0, 0
    for p, x in enumerate(order):
        if par[x] == -1:
            act = ACT_INIT
        elif p > 0 and order[p - 1] == par[x]:
            act = ACT_CONTINUE
        elif children[par[x]][-1] == x:
            act = ACT_POP
            stack_len -= 1
        else:
            act = ACT_TOP
        if len(children[x]) >= 2:
            act |= ACT_PUSH
            stack_len += 1
            max_stack = max(max_stack, stack_len)
        if not children[x]:
            act |= ACT_LEAF
        action.append(act)

    nodepath = np.full((n, MAX_PATH), -1, dtype=np.int32)
    for i in range(n):
        chain, j = [], i
        while j != -1:
            chain.append(j)
            j = par[j]
        chain.reverse()
        nodepath[i, : len(chain)] = chain[:MAX_PATH]
    return {
        "depth": np.asarray(depth, dtype=np.int32),
        "order": np.asarray(order, dtype=np.int32),
        "action": np.asarray(action, dtype=np.int32),
        "nodepath": nodepath,
        "max_stack": max_stack,
        "size": np.asarray(size, dtype=np.int32),
    }


def stack_bound(max_nodes: int) -> int:
    """Largest stack the heavy-last order can need for a tree of max_nodes nodes.

    A push at node P is live only while a non-last child subtree of P is being
    walked, and P's last child is at least as large, so k nested pushes need a
    subtree of >= 2^(k+1) - 1 nodes."""
    k = 0
    while (1 << (k + 2)) - 1 <= max_nodes:
        k += 1
    return k

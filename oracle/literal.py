"""The gated delta rule as a literal matrix product, for tiny pins.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

``literal_rule`` evaluates  S' = a * S @ (I - b k k^T) + b * v k^T  with an
explicit D_k x D_k matrix, exactly as the expression reads, so that the row
form in ``gdn_oracle.c`` (which never forms I - b k k^T) is checked against an
independent evaluation.  ``path_replay`` walks a node's ancestors and applies
the literal rule root-first, one node at a time.
"""
from __future__ import annotations

import numpy as np


def literal_rule(S, k, v, a, b):
    S = np.asarray(S, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    eye = np.eye(len(k))
    return a * S @ (eye - b * np.outer(k, k)) + b * np.outer(v, k)


def path_of(parent, node):
    path = []
    while node != -1:
        path.append(int(node))
        node = int(parent[node])
    return path[::-1]


def path_replay(parent, node, S0, k, v, a, b):
    """State of ``node`` for one head: literal rule over its root-to-node path.
    k [n, dk], v [n, dv], a/b [n] for this head; S0 [dv, dk]."""
    S = np.asarray(S0, dtype=np.float64)
    for j in path_of(parent, node):
        S = literal_rule(S, k[j], v[j], float(a[j]), float(b[j]))
    return S

"""Draft-tree metadata (oracle; test infrastructure only).

"Luce DFlash" README, "How it works": the draft tree is given by parent pointers and
one target forward scores every node under a causal mask derived from them.  Reading
taken: node 0 is the root (parent -1) and every other node's parent has a smaller
index (any topological numbering; the pages' DFS order is one of them).
"""
from __future__ import annotations

import numpy as np


def validate_tree(parent, n: int) -> None:
    parent = np.asarray(parent)
    if n < 1 or n > len(parent):
        raise ValueError(f"n_nodes={n} out of range")
    if int(parent[0]) != -1:
        raise ValueError("node 0 must be the root (parent -1)")
    for i in range(1, n):
        p = int(parent[i])
        if not (0 <= p < i):
            raise ValueError(f"parent[{i}]={p} is not an earlier node")


def depths(parent, n: int) -> np.ndarray:
    d = np.zeros(n, dtype=np.int64)
    for i in range(1, n):
        d[i] = d[int(parent[i])] + 1
    return d


def root_path(parent, i: int) -> list:
    """Nodes from the root down to ``i`` (inclusive)."""
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[i])
    return out[::-1]


def ancestor_matrix(parent, n: int) -> np.ndarray:
    """``A[i, j]`` is True iff node j lies on the root path of node i (self included)."""
    A = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in root_path(parent, i):
            A[i, j] = True
    return A


def validate_path(parent, n: int, path, L: int) -> None:
    """An accepted path is a root path: it starts at the root and each entry is a child of
    the previous one ("Luce DFlash" README, "How it works": after accept, the state is the
    committed prefix).  An empty path (L = 0) accepts nothing and is valid."""
    path = np.asarray(path)
    if L < 0 or L > n or L > len(path):
        raise ValueError(f"path length {L} out of range")
    if L > 0 and int(path[0]) != 0:
        raise ValueError("path must start at the root")
    for m in range(1, L):
        a = int(path[m])
        if not (0 <= a < n) or int(parent[a]) != int(path[m - 1]):
            raise ValueError(f"path[{m}]={a} is not a child of path[{m - 1}]")

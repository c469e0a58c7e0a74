"""Greedy tree acceptance and KV compaction (oracle; test infrastructure only).

"Luce DFlash" README, "How it works": one target forward scores every node of the draft
tree; after accept, the recurrent state and the KV cache are restored to the committed
prefix.  "Scope and limits": the verify skeleton stays argmax, and temperature 0 keeps the
committed path exactly greedy.  The pages do not write the acceptance walk out; the
reading taken here:

* argmax of a node's logits: the lowest index holding the largest value; NaN entries are
  never selected; a row with no non-NaN entry gives index 0.
* walk: start at the root.  At accepted node p the target predicts argmax(p); the next
  accepted node is the child c of p (parent[c] == p, c < n) whose draft token equals that
  prediction -- the lowest-index such child if several do -- and the walk stops when no
  child does.  The path lists the accepted nodes, root first; the next token is the
  target's prediction at the last accepted node (the token committed after the accepted
  draft tokens).
* compaction: the K/V rows of the accepted nodes, stored at tree slots T + node, move to
  the consecutive slots T + m (m = position on the path), byte for byte; every other slot
  keeps its bytes.
"""
from __future__ import annotations

import numpy as np

from .delta import bf16_bits_to_f64


def logits_f64(logits, dtype: str) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16) or fp32 logits."""
    if dtype == "bf16":
        return bf16_bits_to_f64(logits)
    if dtype == "f32":
        return np.asarray(logits, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def argmax_rows(logits, dtype: str) -> np.ndarray:
    """Argmax over the last axis with the tie and NaN rules of the module docstring."""
    x = logits_f64(logits, dtype)
    nan = np.isnan(x)
    key = np.where(nan, -np.inf, x)
    m = key.max(axis=-1, keepdims=True)
    cand = (~nan) & (key == m)
    return np.argmax(cand, axis=-1).astype(np.int64)     # first True; 0 when none


def greedy_walk(parent, n: int, tokens, target):
    """Accepted path (root first), its length and the next token for one sequence."""
    parent = np.asarray(parent)
    tokens = np.asarray(tokens)
    target = np.asarray(target)
    path = [0]
    cur = 0
    while True:
        nxt = None
        for c in range(1, n):
            if int(parent[c]) == cur and int(tokens[c]) == int(target[cur]):
                nxt = c
                break
        if nxt is None:
            break
        path.append(nxt)
        cur = nxt
    return path, len(path), int(target[cur])


def tree_accept_greedy(logits, dtype: str, parent, n_nodes, tokens):
    """Batched: returns (target [B][N] int64 with -1 beyond n, path [B][N] with -1 padding,
    path_len [B], next_token [B])."""
    parent = np.asarray(parent)
    B, N = parent.shape
    tgt = np.full((B, N), -1, dtype=np.int64)
    path = np.full((B, N), -1, dtype=np.int64)
    plen = np.zeros(B, dtype=np.int64)
    nxt = np.zeros(B, dtype=np.int64)
    for b in range(B):
        n = int(n_nodes[b])
        tgt[b, :n] = argmax_rows(np.asarray(logits)[b, :n], dtype)
        p, L, t = greedy_walk(parent[b], n, np.asarray(tokens)[b], tgt[b])
        path[b, :L] = p
        plen[b] = L
        nxt[b] = t
    return tgt, path, plen, nxt


def kv_compact(cache, n_past, path, path_len) -> np.ndarray:
    """A copy of ``cache`` ([B][Hkv][Tcap][row bytes], uint8) after moving each sequence's
    accepted tree rows T + path[m] to T + m, reading every source from the original."""
    cache = np.asarray(cache)
    out = cache.copy()
    for b in range(cache.shape[0]):
        T = int(n_past[b])
        for m in range(int(path_len[b])):
            out[b, :, T + m] = cache[b, :, T + int(path[b][m])]
    return out

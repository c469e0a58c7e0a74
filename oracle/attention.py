"""Tree-masked softmax attention over a quantised KV cache -- oracle, float64.

Sources: "Luce DFlash" README, "How it works" (one target forward verifies the whole
tree through a causal mask derived from parent pointers), "Architecture note" (24 query
heads share 4 KV heads, head length 256), the long-context results and flag table
(sliding-window flash attention, ``--fa-window N``, 0 = full attention) and
"Asymmetric K/V quantization" (K and V each stored as Q8_0 or Q4_0; default q8_0).

Readings taken where the pages are silent:

* Block formats follow the GGUF convention.  Q8_0 block (34 bytes): little-endian fp16
  scale d, then 32 int8 q; element e = d * q[e].  Q4_0 block (18 bytes): fp16 scale d,
  then 16 bytes qs; element e < 16 = d * ((qs[e] & 15) - 8), element e + 16 =
  d * ((qs[e] >> 4) - 8).  A cache row (one slot of one KV head) is D/32 consecutive
  blocks.
* Query head h reads KV head ``h // (Hq // Hkv)``.
* Committed slot t < T sits at position t; tree node j sits in slot T + j at position
  T + depth(j).  Query node i (position T + depth(i)) sees committed slot t iff W == 0 or
  (T + depth(i)) - t < W, and tree slot T + j iff j is on i's root path and (W == 0 or
  depth(i) - depth(j) < W): the W most recent positions, itself included.
* Scores are ``scale * <q, k>``; the output is the softmax-weighted sum of V rows, and
  lse = log(sum(exp(score))) in natural log.
"""
from __future__ import annotations

import numpy as np

from .delta import bf16_bits_to_f64
from .tree import ancestor_matrix, depths, validate_tree

Q8_0_BLOCK_BYTES = 34
Q4_0_BLOCK_BYTES = 18


def _scales(blocks: np.ndarray) -> np.ndarray:
    lo = blocks[..., 0].astype(np.uint16)
    hi = blocks[..., 1].astype(np.uint16)
    return (lo | (hi << 8)).view(np.float16).astype(np.float64)


def dequant_q8_0(rows: np.ndarray) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    nb = rows.shape[-1] // Q8_0_BLOCK_BYTES
    blk = rows.reshape(*rows.shape[:-1], nb, Q8_0_BLOCK_BYTES)
    d = _scales(blk)
    q = blk[..., 2:].view(np.int8).astype(np.float64)
    return (d[..., None] * q).reshape(*rows.shape[:-1], nb * 32)


def dequant_q4_0(rows: np.ndarray) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    nb = rows.shape[-1] // Q4_0_BLOCK_BYTES
    blk = rows.reshape(*rows.shape[:-1], nb, Q4_0_BLOCK_BYTES)
    d = _scales(blk)
    qs = blk[..., 2:]
    nib = np.concatenate([qs & 15, qs >> 4], axis=-1).astype(np.float64) - 8.0
    return (d[..., None] * nib).reshape(*rows.shape[:-1], nb * 32)


def dequant_rows(rows: np.ndarray, kv_type: str) -> np.ndarray:
    if kv_type == "q8_0":
        return dequant_q8_0(rows)
    if kv_type == "q4_0":
        return dequant_q4_0(rows)
    raise ValueError(kv_type)


def visible_slots(T: int, i: int, dep: np.ndarray, anc: np.ndarray, n: int, W: int) -> np.ndarray:
    """Cache slots query node i attends to, in increasing order."""
    pi = T + int(dep[i])
    lo = 0 if W == 0 else max(0, pi - W + 1)
    committed = np.arange(lo, T) if lo < T else np.arange(0)
    tree = [T + j for j in range(n) if anc[i, j] and (W == 0 or int(dep[i]) - int(dep[j]) < W)]
    return np.concatenate([committed, np.array(tree, dtype=np.int64)]).astype(np.int64)


def _attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    s = scale * (qrows @ K.T)                    # [rows][slots]
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ V) / l, (m + np.log(l))[:, 0]


def attn_tree_verify(q, k_cache, v_cache, k_type: str, v_type: str, n_past, parent, n_nodes,
                     window: int, scale: float, Hkv: int):
    """All outputs.  Shapes: q bf16 bits ``[B][N][Hq][D]``; caches uint8
    ``[B][Hkv][Tcap][row_bytes]``.  Returns float64 ``out [B][N][Hq][D]`` and
    ``lse [B][N][Hq]`` (rows at or beyond n_nodes[b] are zero)."""
    qf = bf16_bits_to_f64(q)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, N, Hq))
    for b in range(B):
        n, T = int(n_nodes[b]), int(n_past[b])
        validate_tree(parent[b], n)
        dep = depths(parent[b], n)
        anc = ancestor_matrix(parent[b], n)
        vis = [visible_slots(T, i, dep, anc, n, window) for i in range(n)]
        lo = min(int(v.min()) for v in vis)
        for kvh in range(Hkv):
            K = dequant_rows(k_cache[b, kvh, lo:T + n], k_type)
            V = dequant_rows(v_cache[b, kvh, lo:T + n], v_type)
            for i in range(n):
                idx = vis[i] - lo
                heads = slice(kvh * G, (kvh + 1) * G)
                o, l = _attend(qf[b, i, heads], K[idx], V[idx], scale)
                out[b, i, heads] = o
                lse[b, i, heads] = l
    return out, lse


def attn_tree_verify_rows(q, k_cache, v_cache, k_type: str, v_type: str, n_past, parent, n_nodes,
                          window: int, scale: float, Hkv: int, rows, chunk: int = 16384):
    """Selected outputs only, for caches too large to dequantise whole.  ``rows`` is a list
    of (b, i, h); returns float64 ``out [len(rows)][D]`` and ``lse [len(rows)]``.  Each row
    is the same softmax as above, accumulated over chunks of its visible slots."""
    qf = bf16_bits_to_f64(q)
    Hq, D = qf.shape[2], qf.shape[3]
    G = Hq // Hkv
    outs = np.zeros((len(rows), D))
    lses = np.zeros(len(rows))
    cache = {}
    for r, (b, i, h) in enumerate(rows):
        n, T = int(n_nodes[b]), int(n_past[b])
        if b not in cache:
            validate_tree(parent[b], n)
            cache[b] = (depths(parent[b], n), ancestor_matrix(parent[b], n))
        dep, anc = cache[b]
        idx = visible_slots(T, i, dep, anc, n, window)
        kvh = h // G
        qv = qf[b, i, h]
        # exact two-pass softmax: scores first (max), then weights
        scores = np.empty(len(idx))
        for c0 in range(0, len(idx), chunk):
            K = dequant_rows(k_cache[b, kvh, idx[c0:c0 + chunk]], k_type)
            scores[c0:c0 + chunk] = scale * (K @ qv)
        m = scores.max()
        p = np.exp(scores - m)
        acc = np.zeros(D)
        for c0 in range(0, len(idx), chunk):
            V = dequant_rows(v_cache[b, kvh, idx[c0:c0 + chunk]], v_type)
            acc += p[c0:c0 + chunk] @ V
        l = p.sum()
        outs[r] = acc / l
        lses[r] = m + np.log(l)
    return outs, lses


def visibility_mask(T: int, dep: np.ndarray, anc: np.ndarray, n: int, W: int, lo: int) -> np.ndarray:
    """``M[i, s]`` is True iff query node i sees cache slot ``lo + s`` for slots lo .. T+n-1
    (the window and ancestry rule of the module docstring, as a dense mask)."""
    slots = np.arange(lo, T + n)
    pos = np.where(slots < T, slots, 0).astype(np.int64)
    M = np.zeros((n, len(slots)), dtype=bool)
    for i in range(n):
        pi = T + int(dep[i])
        committed = slots < T
        if W:
            committed &= (pi - pos) < W
        M[i] = committed
        for j in range(n):
            if anc[i, j] and (W == 0 or int(dep[i]) - int(dep[j]) < W):
                M[i, T + j - lo] = True
    return M


def attn_tree_verify_dense(q, k_cache, v_cache, k_type: str, v_type: str, n_past, parent, n_nodes,
                           window: int, scale: float, Hkv: int, chunk: int = 32768):
    """The same outputs as ``attn_tree_verify``, computed as one masked softmax per KV head
    over the union of the slots any node sees: scores of every (node, query head) row against
    the union, invisible slots set to -inf, then softmax-weighted V.  Dequantised K and V are
    taken in chunks of slots, so caches of 10^5 slots fit in memory; the softmax is exact
    (scores of the whole union are kept, then one max, one exp, one weighted sum)."""
    qf = bf16_bits_to_f64(q)
    B, N, Hq, D = qf.shape
    G = Hq // Hkv
    out = np.zeros((B, N, Hq, D))
    lse = np.zeros((B, N, Hq))
    for b in range(B):
        n, T = int(n_nodes[b]), int(n_past[b])
        validate_tree(parent[b], n)
        dep = depths(parent[b], n)
        anc = ancestor_matrix(parent[b], n)
        lo = 0 if window == 0 else max(0, T + int(dep.min()) - window + 1)
        M = visibility_mask(T, dep, anc, n, window, lo)          # [n][slots]
        S = T + n - lo
        for kvh in range(Hkv):
            heads = slice(kvh * G, (kvh + 1) * G)
            Q = qf[b, :n, heads].reshape(n * G, D)                # row r = node r // G, head r % G
            vis = np.repeat(M, G, axis=0)
            s = np.empty((n * G, S))
            for c0 in range(0, S, chunk):
                K = dequant_rows(k_cache[b, kvh, lo + c0:lo + min(S, c0 + chunk)], k_type)
                s[:, c0:c0 + K.shape[0]] = scale * (Q @ K.T)
            s[~vis] = -np.inf
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            acc = np.zeros((n * G, D))
            for c0 in range(0, S, chunk):
                V = dequant_rows(v_cache[b, kvh, lo + c0:lo + min(S, c0 + chunk)], v_type)
                acc += p[:, c0:c0 + V.shape[0]] @ V
            l = p.sum(axis=1, keepdims=True)
            out[b, :n, heads] = (acc / l).reshape(n, G, D)
            lse[b, :n, heads] = (m + np.log(l))[:, 0].reshape(n, G)
    return out, lse

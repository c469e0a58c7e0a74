"""Gated delta-rule (linear attention) over a draft tree -- oracle, float64.

Sources: "Luce DFlash" README, "Architecture note" (three of every four layers are
Gated DeltaNet: linear attention with a learned recurrence and a recurrent state cache)
and "How it works" (the tree-mode gated-delta-net kernels run the recurrence along each
node's parent chain; after accept the state is restored to the committed prefix);
PR #606 "SpecLA factor-capture speculative decoding", "Paper mapping" (a chain is a
degenerate tree).

Readings taken where the pages are silent:

* The recurrence is the standard gated delta rule, with the state S (dk x dv) mapping
  keys to values, the decay g applied multiplicatively, and the output read after the
  update::

      u_i     = S_p^T k_i
      delta_i = beta_i * (v_i - g_i * u_i)
      S_i     = g_i * S_p + k_i delta_i^T
      o_i     = scale * S_i^T q_i

  where p is node i's parent and S_{-1} is the committed state S0.
* Value head h reads key head ``h // (Hv // Hk)`` ("contiguous", the default) or
  ``h % Hk`` ("tiled").
* Memory layout of the state: ``state[b][h][c][r] = S[r][c]`` (one row of dk keys per
  value channel c).
* q and k arrive already normalised; nothing here normalises them.
"""
from __future__ import annotations

import numpy as np

from .tree import validate_tree, validate_path


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def as_f64(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def key_head(h: int, Hk: int, Hv: int, head_group: str = "contiguous") -> int:
    if head_group == "contiguous":
        return h // (Hv // Hk)
    if head_group == "tiled":
        return h % Hk
    raise ValueError(head_group)


def lin_tree_verify(q, k, v, g, beta, state, parent, n_nodes, scale: float, dtype: str = "f32",
                    head_group: str = "contiguous", return_states: bool = False):
    """Score every tree node of every sequence through one linear-attention layer.

    Shapes: q, k ``[B][N][Hk][dk]``; v ``[B][N][Hv][dv]``; g, beta ``[B][N][Hv]``;
    state ``[B][Hv][dv][dk]``; parent ``[B][N]``; n_nodes ``[B]``.

    Returns ``(out, delta)`` as float64 ``[B][N][Hv][dv]`` (rows at or beyond n_nodes[b]
    are zero) and, if asked, ``states[b][h][i]`` = S_i as a dk x dv array.
    """
    qf, kf, vf = as_f64(q, dtype), as_f64(k, dtype), as_f64(v, dtype)
    gf, bf = as_f64(g, dtype), as_f64(beta, dtype)
    S0all = np.asarray(state, dtype=np.float32).astype(np.float64)
    B, N, Hk, dk = qf.shape
    Hv, dv = vf.shape[2], vf.shape[3]
    out = np.zeros((B, N, Hv, dv))
    delta = np.zeros((B, N, Hv, dv))
    states = [[None] * Hv for _ in range(B)] if return_states else None
    for b in range(B):
        n = int(n_nodes[b])
        validate_tree(parent[b], n)
        for h in range(Hv):
            kh = key_head(h, Hk, Hv, head_group)
            S0 = S0all[b, h].T                      # dk x dv
            S = [None] * n
            for i in range(n):
                p = int(parent[b][i])
                Sp = S0 if p < 0 else S[p]
                ki, qi = kf[b, i, kh], qf[b, i, kh]
                u = Sp.T @ ki
                d = bf[b, i, h] * (vf[b, i, h] - gf[b, i, h] * u)
                S[i] = gf[b, i, h] * Sp + np.outer(ki, d)
                out[b, i, h] = scale * (S[i].T @ qi)
                delta[b, i, h] = d
            if return_states:
                states[b][h] = S
    if return_states:
        return out, delta, states
    return out, delta


def lin_commit_replay(state, path, path_len, k, v, g, beta, parent, n_nodes, dtype: str = "f32",
                      head_group: str = "contiguous") -> np.ndarray:
    """The committed state after accepting ``path``: the recurrence replayed from S0 over
    the accepted tokens alone, in path order.  Returns float64 ``[B][Hv][dv][dk]``."""
    kf, vf = as_f64(k, dtype), as_f64(v, dtype)
    gf, bf = as_f64(g, dtype), as_f64(beta, dtype)
    S0all = np.asarray(state, dtype=np.float32).astype(np.float64)
    B, _, Hk, dk = kf.shape
    Hv = vf.shape[2]
    new = np.empty_like(S0all)
    for b in range(B):
        n, L = int(n_nodes[b]), int(path_len[b])
        validate_tree(parent[b], n)
        validate_path(parent[b], n, path[b], L)
        for h in range(Hv):
            kh = key_head(h, Hk, Hv, head_group)
            S = S0all[b, h].T.copy()
            for m in range(L):
                a = int(path[b][m])
                ka = kf[b, a, kh]
                d = bf[b, a, h] * (vf[b, a, h] - gf[b, a, h] * (S.T @ ka))
                S = gf[b, a, h] * S + np.outer(ka, d)
            new[b, h] = S.T
    return new


def lin_chain_recurrence(q, k, v, g, beta, S0, scale: float):
    """The sequential recurrence over one token list (a chain), for one head.

    q, k ``[L][dk]``, v ``[L][dv]``, g, beta ``[L]``, S0 ``dk x dv`` (float64).
    Returns (outputs ``[L][dv]``, final state)."""
    S = np.array(S0, dtype=np.float64)
    outs = []
    for t in range(len(g)):
        d = beta[t] * (v[t] - g[t] * (S.T @ k[t]))
        S = g[t] * S + np.outer(k[t], d)
        outs.append(scale * (S.T @ q[t]))
    return np.array(outs), S


def lin_tree_verify_commit(state, prev, q, k, v, g, beta, parent, n_nodes, scale: float, dtype: str = "f32",
                           head_group: str = "contiguous"):
    """One verify step that first commits the previous step's accepted path.

    PR #606 "SpecLA factor-capture speculative decoding" (the factors captured during verify
    are flushed into the raw state on commit; the pending-bank variant applies them while
    the next verify loads the state).  Reading taken: the previous step's commit is the
    plain commit of its accepted path (``lin_commit_replay``), the state is stored as fp32,
    and this step's verify starts from that stored committed state.

    ``prev`` = (path, path_len, k, v, g, beta, parent, n_nodes) of the previous step.
    Returns ``(committed_state, out, delta)``: the committed state rounded to fp32 as the
    stored state (float64 array of fp32 values) and this step's outputs and deltas."""
    path, path_len, pk, pv, pg, pbeta, pparent, pn = prev
    committed = lin_commit_replay(state, path, path_len, pk, pv, pg, pbeta, pparent, pn, dtype, head_group)
    stored = committed.astype(np.float32)
    out, delta = lin_tree_verify(q, k, v, g, beta, stored, parent, n_nodes, scale, dtype, head_group)
    return stored.astype(np.float64), out, delta


def lin_tree_verify_bank(state, pending, q, k, v, g, beta, parent, n_nodes, scale: float, dtype: str = "f32",
                         head_group: str = "contiguous"):
    """One verify step with several accepted steps still pending.

    PR #606 "SpecLA factor-capture speculative decoding": "CLI" (the fused commit is on by
    default) and the review comment on the pending bank (a pending count of accepted
    factors, flushed into the raw state).  Reading taken: the pending steps are committed in
    acceptance order, each exactly as a separate commit of its accepted path would
    (``lin_commit_replay``, its result stored as fp32), and this step's verify starts from
    the state they reach.  How many steps stay pending before a flush does not change any
    value: it only decides when the state is written.

    ``pending`` = the steps accepted since the state was last stored, oldest first, each
    (path, path_len, k, v, g, beta, parent, n_nodes) of that step.  Returns
    ``(committed_state, out, delta)`` as ``lin_tree_verify_commit`` does."""
    S = np.asarray(state, dtype=np.float32).astype(np.float64)
    for prev in pending:
        path, path_len, pk, pv, pg, pbeta, pparent, pn = prev
        S = lin_commit_replay(S, path, path_len, pk, pv, pg, pbeta, pparent, pn, dtype, head_group)
        S = S.astype(np.float32).astype(np.float64)
    out, delta = lin_tree_verify(q, k, v, g, beta, S.astype(np.float32), parent, n_nodes, scale, dtype, head_group)
    return S, out, delta

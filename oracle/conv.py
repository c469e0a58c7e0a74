"""Causal short convolution over a draft tree -- oracle, float64 (test infrastructure only).

Sources: "Luce DFlash" README, "How it works": the recurrent state rolled back after
acceptance holds, besides the delta-rule state, the convolution window; the tree-aware
convolution takes each node's window of earlier inputs along its parent chain in the
draft tree, not in node (DFS) order.  "Architecture note": the Gated DeltaNet layers keep
a recurrent state cache (which, in the models the pages run, includes that window).

The pages do not write the convolution out.  The reading taken:

* Per channel c, a causal depthwise convolution of width K over the layer's input
  sequence, no bias::

      y_i[c] = sum_{k=0}^{K-1} w[c][k] * u_{i,k}[c]

  where u_{i,K-1} is node i's own input, u_{i,K-2} its parent's, and so on up the root
  path; positions above the root come from the committed window ``state`` (K-1 earlier
  inputs per channel, oldest first: the most recent committed input is
  ``state[K-2]``).  On a chain this is ordinary causal 1-D convolution.
* Optionally the output passes through SiLU, v * sigmoid(v) (``activation`` = "silu").
* Commit along an accepted root path a_0 .. a_{L-1}: the new window is the last K-1
  inputs of (committed window, x[a_0], ..., x[a_{L-1}]).  L = 0 leaves it unchanged.
* K is a model parameter the pages do not state; it is an argument here.
"""
from __future__ import annotations

import numpy as np

from .delta import as_f64


def conv_tree_verify(x, dtype: str, weight, state, parent, n_nodes, activation: str = "none") -> np.ndarray:
    """x [B][N][C] (bf16 bits or f32), weight [C][K], state [B][K-1][C] -> y [B][N][C] float64
    (rows at or beyond n_nodes[b] are left at 0)."""
    xf = as_f64(x, dtype)
    w = np.asarray(weight, dtype=np.float64)
    st = np.asarray(state, dtype=np.float64)
    parent = np.asarray(parent)
    B, N, C = xf.shape
    K = w.shape[1]
    assert st.shape == (B, K - 1, C), (st.shape, (B, K - 1, C))
    y = np.zeros((B, N, C))
    for b in range(B):
        for i in range(int(n_nodes[b])):
            acc = np.zeros(C)
            node = i
            above = 0                      # steps taken above the root, into the window
            for k in range(K - 1, -1, -1):
                if node >= 0:
                    u = xf[b, node]
                    node = int(parent[b, node]) if node > 0 else -1
                else:
                    above += 1
                    u = st[b, K - 1 - above]
                acc = acc + w[:, k] * u
            if activation == "silu":
                acc = acc / (1.0 + np.exp(-acc))
            elif activation != "none":
                raise ValueError(activation)
            y[b, i] = acc
    return y


def conv_tree_commit(x, dtype: str, state, path, path_len) -> np.ndarray:
    """The committed window after accepting each sequence's path: [B][K-1][C] float64."""
    xf = as_f64(x, dtype)
    st = np.asarray(state, dtype=np.float64)
    B, Km1, C = st.shape
    out = st.copy()
    for b in range(B):
        L = int(path_len[b])
        seq = [st[b, j] for j in range(Km1)] + [xf[b, int(path[b][m])] for m in range(L)]
        out[b] = np.stack(seq[len(seq) - Km1:]) if Km1 > 0 else out[b]
    return out

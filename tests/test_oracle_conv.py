"""Pins of the tree-aware causal convolution oracle (oracle/conv.py) -- CPU only.

* a hand-worked tree (tests/golden/conv_handworked.json), including a sibling branch whose
  window must skip the sibling (the node-order mistake the pages warn about);
* a chain equals PyTorch's grouped 1-D convolution (float64) over the committed window
  followed by the chain's inputs;
* relabeling invariance (any topological numbering gives the same per-node outputs);
* commit followed by one more token equals the chain convolution over everything;
* SiLU: silu(v) - silu(-v) = v and silu(0) = 0.
"""
import json
import os

import numpy as np
import torch

import oracle
from workloads import tree_ddtree, tree_chain, pad_trees, random_root_leaf_path

GOLD = os.path.join(os.path.dirname(__file__), "golden", "conv_handworked.json")


def test_handworked_tree_and_commits():
    g = json.load(open(GOLD))
    x = np.array(g["x"], np.float32)[None]
    parent = np.array([g["parent"]], np.int32)
    n = np.array([len(g["parent"])], np.int32)
    y = oracle.conv_tree_verify(x, "f32", np.array(g["weight"], np.float32), np.array([g["state"]], np.float32),
                                parent, n)
    assert np.array_equal(y[0], np.array(g["y"], np.float64))
    for c in g["commits"]:
        L = len(c["path"])
        path = np.array([c["path"] + [-1] * (4 - L)], np.int32)
        st = oracle.conv_tree_commit(x, "f32", np.array([g["state"]], np.float32), path, np.array([L]))
        assert np.array_equal(st[0], np.array(c["state"], np.float64)), c["note"]


def _chain_conv_torch(state, xs, w):
    """[K-1][C] window + [T][C] inputs, weight [C][K] -> [T][C] via torch grouped conv1d."""
    seq = torch.from_numpy(np.concatenate([state, xs], 0).T[None].copy())        # [1][C][K-1+T]
    wt = torch.from_numpy(np.asarray(w, np.float64)[:, None, :].copy())          # [C][1][K]
    return torch.nn.functional.conv1d(seq, wt, groups=w.shape[0])[0].T.numpy()   # [T][C]


def test_chain_equals_grouped_conv1d():
    rng = np.random.default_rng(0)
    for K in (2, 3, 4, 6):
        C, n = 7, 9
        x = rng.standard_normal((1, n, C)).astype(np.float32)
        w = rng.standard_normal((C, K)).astype(np.float32)
        st = rng.standard_normal((1, K - 1, C)).astype(np.float32)
        y = oracle.conv_tree_verify(x, "f32", w, st, tree_chain(n)[None], np.array([n]))
        ref = _chain_conv_torch(st[0].astype(np.float64), x[0].astype(np.float64), w)
        np.testing.assert_allclose(y[0], ref, rtol=1e-12, atol=1e-12)


def test_relabeling_invariance():
    rng = np.random.default_rng(1)
    p = tree_ddtree(rng, budget=22)
    n = len(p)
    # a second topological numbering: breadth-first order of the same tree
    kids = [[c for c in range(1, n) if p[c] == q] for q in range(n)]
    order, frontier = [0], [0]
    while frontier:
        nxt = [c for q in frontier for c in kids[q]]
        order += nxt
        frontier = nxt
    new_of = {old: new for new, old in enumerate(order)}
    p2 = np.array([-1] + [new_of[int(p[old])] for old in order[1:]], np.int32)
    C, K = 5, 4
    x = rng.standard_normal((1, n, C)).astype(np.float32)
    x2 = x[:, order]
    w = rng.standard_normal((C, K)).astype(np.float32)
    st = rng.standard_normal((1, K - 1, C)).astype(np.float32)
    y = oracle.conv_tree_verify(x, "f32", w, st, p[None], np.array([n]))
    y2 = oracle.conv_tree_verify(x2, "f32", w, st, p2[None], np.array([n]))
    np.testing.assert_allclose(y2[0], y[0][order], rtol=1e-12, atol=1e-12)


def test_commit_then_next_token_equals_chain_conv():
    rng = np.random.default_rng(2)
    C, K = 6, 4
    p = tree_ddtree(rng, budget=22)
    n = len(p)
    for trial in range(5):
        x = rng.standard_normal((1, n, C)).astype(np.float32)
        w = rng.standard_normal((C, K)).astype(np.float32)
        st = rng.standard_normal((1, K - 1, C)).astype(np.float32)
        path = random_root_leaf_path(rng, p, n)[: 1 + trial]
        L = len(path)
        new = oracle.conv_tree_commit(x, "f32", st, path[None], np.array([L]))
        nxt = rng.standard_normal((1, 1, C)).astype(np.float32)
        y = oracle.conv_tree_verify(nxt, "f32", w, new.astype(np.float32), np.array([[-1]], np.int32), np.array([1]))
        ref = _chain_conv_torch(st[0].astype(np.float64), np.concatenate([x[0, path], nxt[0]], 0).astype(np.float64), w)
        np.testing.assert_allclose(y[0, 0], ref[-1], rtol=1e-12, atol=1e-12)


def test_silu_identity():
    rng = np.random.default_rng(3)
    C, K = 4, 2
    x = rng.standard_normal((1, 3, C)).astype(np.float32) * 4
    w = rng.standard_normal((C, K)).astype(np.float32)
    st = rng.standard_normal((1, K - 1, C)).astype(np.float32)
    p = tree_chain(3)[None]
    lin = oracle.conv_tree_verify(x, "f32", w, st, p, np.array([3]))
    pos = oracle.conv_tree_verify(x, "f32", w, st, p, np.array([3]), activation="silu")
    neg = oracle.conv_tree_verify(-x, "f32", w, -st, p, np.array([3]), activation="silu")
    # the convolution is linear, so negating inputs and window negates v exactly
    np.testing.assert_allclose(pos[0] - neg[0], lin[0], rtol=1e-12, atol=1e-12)
    z = oracle.conv_tree_verify(np.zeros_like(x), "f32", w, np.zeros_like(st), p, np.array([3]), activation="silu")
    assert np.all(z == 0.0)

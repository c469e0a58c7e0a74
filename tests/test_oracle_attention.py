"""Pins for the tree-attention oracle (CPU only).

Checks against hand-decoded block fixtures, PyTorch's scaled-dot-product attention
(float64, CPU) for chains with causal and sliding-window masks, brute force over each
node's root path, and closed forms (window 1, empty history).
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import (attn_tree_verify, attn_tree_verify_rows, attn_tree_verify_dense, dequant_q8_0, dequant_q4_0,
                    dequant_rows, root_path, depths)
from oracle.delta import bf16_bits_to_f64
from workloads import (gen_attn, trees_for, tree_chain, tree_ddtree, quantize_q8_0, quantize_q4_0,
                       f32_to_bf16_bits, row_bytes)


def test_block_fixtures(golden_dir):
    with open(os.path.join(golden_dir, "kv_blocks_handworked.json")) as f:
        gj = json.load(f)
    b8 = np.frombuffer(bytes.fromhex(gj["q8_0"]["hex"]), np.uint8)
    b4 = np.frombuffer(bytes.fromhex(gj["q4_0"]["hex"]), np.uint8)
    assert np.array_equal(dequant_q8_0(b8), np.array(gj["q8_0"]["expect"], float))
    assert np.array_equal(dequant_q4_0(b4), np.array(gj["q4_0"]["expect"], float))
    # rows are consecutive blocks
    assert np.array_equal(dequant_q8_0(np.concatenate([b8, b8])), np.tile(gj["q8_0"]["expect"], 2))


@pytest.mark.parametrize("kv", ["q8_0", "q4_0"])
def test_quantiser_round_trip(kv):
    """Decoding what the (independent) workload quantiser wrote recovers x to within half a
    quantisation step (Q8_0), or one step (Q4_0, whose code range -8..7 clips the positive
    end by one step), plus the fp16 rounding of the scale."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    q = (quantize_q8_0 if kv == "q8_0" else quantize_q4_0)(x)
    assert q.shape == (64, row_bytes(kv, 256))
    y = dequant_rows(q, kv)
    blk = np.abs(x.reshape(64, 8, 32)).max(-1)
    step = blk / (127.0 if kv == "q8_0" else 8.0)
    err = np.abs(y - x).reshape(64, 8, 32).max(-1)
    frac = 0.5 if kv == "q8_0" else 1.0
    assert np.all(err <= step * frac * (1 + 2 ** -9) + 1e-6)


def _sdpa(qrows, K, V, mask, scale):
    q = torch.from_numpy(qrows)[None]
    k = torch.from_numpy(K)[None]
    v = torch.from_numpy(V)[None]
    m = torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0].numpy()


def _chain_inputs(T, n, window, kv="q8_0", Hq=4, Hkv=2, D=64, seed=0):
    parent = tree_chain(n)
    A = gen_attn(20 + seed, [parent], Hq, Hkv, D, T, kv, kv, window)
    return A


@pytest.mark.parametrize("T,n,window,kv", [(50, 6, 0, "q8_0"), (50, 6, 16, "q8_0"), (40, 5, 3, "q4_0"),
                                           (0, 4, 0, "q8_0"), (30, 7, 31, "q4_0")])
def test_chain_matches_sdpa(T, n, window, kv):
    """A chain is a degenerate tree: node i is token T+i of a plain causal sequence, and a
    sliding window of W keeps keys with (query pos - key pos) < W."""
    A = _chain_inputs(T, n, window, kv)
    out, lse = attn_tree_verify(A.q, A.k_cache, A.v_cache, kv, kv, A.n_past, A.parent, A.n_nodes,
                                window, A.scale, A.Hkv)
    G = A.Hq // A.Hkv
    qf = bf16_bits_to_f64(A.q)
    pos_q = T + np.arange(n)
    pos_k = np.arange(T + n)
    mask = pos_k[None, :] <= pos_q[:, None]
    if window:
        mask &= (pos_q[:, None] - pos_k[None, :]) < window
    for h in range(A.Hq):
        kvh = h // G
        K = dequant_rows(A.k_cache[0, kvh, :T + n], kv)
        V = dequant_rows(A.v_cache[0, kvh, :T + n], kv)
        ref = _sdpa(qf[0, :n, h], K, V, mask, A.scale)
        np.testing.assert_allclose(out[0, :n, h], ref, atol=1e-12)
        s = A.scale * (qf[0, :n, h] @ K.T)
        s = np.where(mask, s, -np.inf)
        ref_lse = np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1)
        np.testing.assert_allclose(lse[0, :n, h], ref_lse, atol=1e-12)


def _tree_inputs(T, window, kv="q8_0", B=1, seed=0, Hq=6, Hkv=2, D=64):
    parents, _ = trees_for(30 + seed, B, "ddtree")
    return gen_attn(30 + seed, parents, Hq, Hkv, D, T, kv, kv, window)


@pytest.mark.parametrize("T,window", [(64, 0), (64, 20), (10, 4), (5, 0)])
def test_tree_equals_per_path_causal(T, window):
    """Brute force: node i attends exactly like the last token of the sequence
    [committed history, root_path(i)] under causal (and window) masking, with tree node j
    placed at position T + depth(j)."""
    A = _tree_inputs(T, window)
    out, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                              A.n_nodes, window, A.scale, A.Hkv)
    qf = bf16_bits_to_f64(A.q)
    n = int(A.n_nodes[0])
    G = A.Hq // A.Hkv
    for i in range(n):
        path = root_path(A.parent[0], i)
        slots = list(range(T)) + [T + j for j in path]
        pos = np.array(list(range(T)) + [T + d for d in range(len(path))])
        pq = pos[-1]
        mask = pos <= pq
        if window:
            mask &= (pq - pos) < window
        for h in range(A.Hq):
            kvh = h // G
            K = dequant_rows(A.k_cache[0, kvh, slots], "q8_0")
            V = dequant_rows(A.v_cache[0, kvh, slots], "q8_0")
            ref = _sdpa(qf[0, i:i + 1, h], K, V, mask[None, :], A.scale)
            np.testing.assert_allclose(out[0, i, h], ref[0], atol=1e-12)


def test_window_one_returns_own_value():
    """W = 1: each node sees only itself, so o_i is its own dequantised V row exactly."""
    A = _tree_inputs(33, 1, kv="q4_0")
    out, lse = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q4_0", "q4_0", A.n_past, A.parent,
                                A.n_nodes, 1, A.scale, A.Hkv)
    G = A.Hq // A.Hkv
    qf = bf16_bits_to_f64(A.q)
    for i in range(int(A.n_nodes[0])):
        for h in range(A.Hq):
            V = dequant_rows(A.v_cache[0, h // G, 33 + i], "q4_0")
            K = dequant_rows(A.k_cache[0, h // G, 33 + i], "q4_0")
            assert np.array_equal(out[0, i, h], V)
            np.testing.assert_allclose(lse[0, i, h], A.scale * qf[0, i, h] @ K, rtol=1e-14)


def test_root_alone_without_history():
    A = _tree_inputs(0, 0)
    out, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                              A.n_nodes, 0, A.scale, A.Hkv)
    G = A.Hq // A.Hkv
    for h in range(A.Hq):
        assert np.array_equal(out[0, 0, h], dequant_rows(A.v_cache[0, h // G, 0], "q8_0"))


def test_wide_window_equals_full():
    A = _tree_inputs(40, 0)
    full, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                               A.n_nodes, 0, A.scale, A.Hkv)
    dmax = int(depths(A.parent[0], int(A.n_nodes[0])).max())
    wide, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                               A.n_nodes, 40 + dmax + 1, A.scale, A.Hkv)
    np.testing.assert_allclose(wide, full, atol=0)
    narrow, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                                 A.n_nodes, 40 + dmax, A.scale, A.Hkv)
    assert not np.allclose(narrow, full)


def test_rows_variant_matches_full():
    A = _tree_inputs(300, 50, B=2, seed=3)
    out, lse = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                                A.n_nodes, 50, A.scale, A.Hkv)
    rows = [(0, 0, 0), (1, 5, 3), (0, 21, 5), (1, 13, 2)]
    o2, l2 = attn_tree_verify_rows(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                                   A.n_nodes, 50, A.scale, A.Hkv, rows, chunk=7)
    for r, (b, i, h) in enumerate(rows):
        np.testing.assert_allclose(o2[r], out[b, i, h], atol=1e-12)
        np.testing.assert_allclose(l2[r], lse[b, i, h], atol=1e-12)


@pytest.mark.parametrize("window,kt,vt,chunk", [(0, "q8_0", "q8_0", 32768), (50, "q8_0", "q4_0", 7),
                                                (1, "q4_0", "q8_0", 64), (3, "q4_0", "q4_0", 5)])
def test_dense_variant_matches_per_node(window, kt, vt, chunk):
    """The dense masked-softmax form (one score matrix per KV head over the union of visible
    slots, taken in slot chunks) equals the per-node form on ragged histories, including a
    sequence with no history and windows of 1 and 3."""
    rng = np.random.default_rng(window + 11)
    parents = [tree_ddtree(rng, budget=22), tree_chain(6), np.array([-1], np.int32)]
    A = gen_attn(33, parents, 6, 2, 64, [300, 0, 17], kt, vt, window)
    ref, rl = attn_tree_verify(A.q, A.k_cache, A.v_cache, kt, vt, A.n_past, A.parent, A.n_nodes, window,
                               A.scale, A.Hkv)
    out, lse = attn_tree_verify_dense(A.q, A.k_cache, A.v_cache, kt, vt, A.n_past, A.parent, A.n_nodes,
                                      window, A.scale, A.Hkv, chunk=chunk)
    np.testing.assert_allclose(out, ref, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_relabeling_invariance():
    """Renumbering the tree (and moving its K/V slots with it) permutes the outputs."""
    A = _tree_inputs(20, 9, seed=4)
    n = int(A.n_nodes[0])
    out, _ = attn_tree_verify(A.q, A.k_cache, A.v_cache, "q8_0", "q8_0", A.n_past, A.parent,
                              A.n_nodes, 9, A.scale, A.Hkv)
    parent = A.parent[0]
    children = [[] for _ in range(n)]
    for i in range(1, n):
        children[parent[i]].append(i)
    order, stack = [], [0]
    while stack:                         # depth-first, last child first
        x = stack.pop()
        order.append(x)
        stack.extend(children[x])
    order = np.array(order)
    new_of = np.empty(n, int)
    new_of[order] = np.arange(n)
    parent2 = np.array([[-1] + [new_of[parent[o]] for o in order[1:]]], np.int32)
    kc, vc = A.k_cache.copy(), A.v_cache.copy()
    kc[:, :, 20:20 + n] = A.k_cache[:, :, 20 + order]
    vc[:, :, 20:20 + n] = A.v_cache[:, :, 20 + order]
    out2, _ = attn_tree_verify(A.q[:, order], kc, vc, "q8_0", "q8_0", A.n_past, parent2, A.n_nodes,
                               9, A.scale, A.Hkv)
    np.testing.assert_allclose(out2[0], out[0, order], atol=1e-12)

"""The benchmark's measurement model, checked on small inputs against counts made from first
principles: the bytes a linear verify / commit must move, and the union of KV slots and the
(row, slot) pairs that tree attention must visit under the window rule (a query node at
position T + depth(i) sees committed slot t iff W = 0 or T + depth(i) - t < W, and tree node j
iff j is on its root path and (W = 0 or depth(i) - depth(j) < W)).  CPU only."""
import numpy as np
import pytest

import bench
from workloads import gen_attn, gen_lin, tree_chain, tree_ddtree, random_root_leaf_path, pad_trees


def _depths(parent, n):
    dep = [0] * n
    for i in range(1, n):
        dep[i] = dep[int(parent[i])] + 1
    return dep


def _ancestors(parent, i):
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[i]) if i > 0 else -1
    return out


def _small_lin(dtype):
    rng = np.random.default_rng(5)
    parents = [tree_ddtree(rng, budget=7), tree_chain(3)]
    parent, n = pad_trees(parents)
    paths = [random_root_leaf_path(rng, parent[0], int(n[0])), np.arange(2, dtype=np.int32)]
    return gen_lin(77, parents, paths, 2, 4, 16, 32, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_linear_bytes(dtype):
    L = _small_lin(dtype)
    e = 2 if dtype == "bf16" else 4
    B, Hv, dv, dk = L.state.shape
    Hk = L.q.shape[2]
    nodes = int(L.n_nodes.sum())
    acc = int(L.path_len.sum())
    # verify: state once; per node q and k rows (Hk x dk), v (Hv x dv), g and beta (Hv), and the
    # fp32 output and captured delta (Hv x dv each); the tree metadata
    verify = B * Hv * dv * dk * 4 + nodes * (2 * Hk * dk * e + Hv * dv * e + 2 * Hv * e + 2 * Hv * dv * 4)
    verify += L.parent.nbytes + L.n_nodes.nbytes
    assert bench.lin_verify_bytes(L) == verify
    # commit: state read and written; per accepted node its k row, captured delta and decay
    commit = 2 * B * Hv * dv * dk * 4 + acc * (Hk * dk * e + Hv * dv * 4 + Hv * e) + L.path.nbytes
    assert bench.lin_commit_bytes(L) == commit
    # fused: the verify's bytes plus the committed state written once and the previous path's inputs
    fused = verify + B * Hv * dv * dk * 4 + acc * (Hk * dk * e + Hv * dv * 4 + Hv * e) + L.path.nbytes
    assert bench.lin_verify_commit_bytes(L) == fused


@pytest.mark.parametrize("window", [0, 1, 3, 6, 50])
def test_attention_bytes_and_flops(window):
    rng = np.random.default_rng(11)
    parents = [tree_ddtree(rng, budget=9, max_depth=5), tree_chain(4), np.array([-1], np.int32)]
    T = [13, 2, 0]
    A = gen_attn(33, parents, 4, 2, 64, T, "q8_0", "q4_0", window, tcap=24)
    B, N, Hq, D = A.q.shape
    rowb = (D // 32) * 34 + (D // 32) * 18
    W = window
    exp_bytes = 0
    exp_pairs = 0
    for b in range(B):
        n, Tb = int(A.n_nodes[b]), int(A.n_past[b])
        par = A.parent[b]
        dep = _depths(par, n)
        union = set()
        for i in range(n):
            pos = Tb + dep[i]
            vis = [t for t in range(Tb) if W == 0 or pos - t < W]
            vis += [Tb + j for j in _ancestors(par, i) if W == 0 or dep[i] - dep[j] < W]
            union.update(vis)
            exp_pairs += Hq * len(vis)
        # the union of visible slots is read once per KV head: every tree slot (each node
        # sees itself) and the committed slots some node sees
        exp_bytes += A.Hkv * len(union) * rowb + n * Hq * (D * 2 + D * 4 + 4)
    assert bench.attn_bytes(A) == exp_bytes
    assert bench.attn_flops(A) == 4.0 * D * exp_pairs

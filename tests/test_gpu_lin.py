"""Parity of the HIP linear-attention verify and commit against the fp64 oracle.

Tolerances: bf16 inputs with an fp32 state -- max |gpu - oracle| <= 2e-3 x RMS(oracle)
per output tensor.  fp32 inputs -- 1e-4 x RMS: the kernel contracts S0 with keys and
queries as split-bf16 products (each operand hi + lo, error <= 2^-16 relative per
product) with fp32 accumulation, so errors of order 1e-5 x RMS are expected.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import lin_to_device, rel_err, valid_rows
from workloads import (workload_tiny_linear, workload_linear_27b, gen_lin, trees_for, tree_chain,
                       tree_ddtree, random_root_leaf_path, rng_for)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-3
TOL_F32 = 1e-4


def run_gpu(L, head_group="contiguous", sentinel=True):
    d = lin_to_device(L)
    B, N = L.parent.shape
    out = torch.full((B, N, L.Hv, L.dv), float("nan"), device="cuda") if sentinel else None
    cap = torch.full((B, N, L.Hv, L.dv), float("nan"), device="cuda") if sentinel else None
    out, cap = tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"],
                                   d["n_nodes"], L.scale, head_group, out=out, cap_delta=cap)
    st = d["state"].clone()
    tvl.lin_tree_commit(st, d["path"], d["path_len"], d["k"], d["g"], cap, head_group)
    torch.cuda.synchronize()
    return out.cpu().numpy(), cap.cpu().numpy(), st.cpu().numpy(), d


def run_oracle(L, head_group="contiguous"):
    o, dl = oracle.lin_tree_verify(L.q, L.k, L.v, L.g, L.beta, L.state, L.parent, L.n_nodes, L.scale,
                                   L.dtype, head_group)
    st = oracle.lin_commit_replay(L.state, L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes,
                                  L.dtype, head_group)
    return o, dl, st


def check(L, tol, head_group="contiguous", label=""):
    out, cap, st, _ = run_gpu(L, head_group)
    ro, rd, rs = run_oracle(L, head_group)
    mask = valid_rows(L.n_nodes, L.parent.shape[1])
    e_out, e_d, e_s = rel_err(out, ro, mask), rel_err(cap, rd, mask), rel_err(st, rs)
    print(f"[lin {label}] out {e_out:.2e}  delta {e_d:.2e}  committed state {e_s:.2e}")
    assert np.isnan(out[~mask]).all() and np.isnan(cap[~mask]).all(), "padding rows were written"
    assert e_out <= tol and e_d <= tol and e_s <= tol
    return out, cap, st


def test_tiny_linear_fp32():
    """1 head, dk=dv=16, fp32, 8-node tree, seeded root-to-leaf path."""
    check(workload_tiny_linear().lin[0], TOL_F32, label="tiny fp32")


def test_linear_27b_width():
    """16 key heads, 48 value heads, dk=dv=128, bf16 inputs, fp32 state, 22-node tree."""
    check(workload_linear_27b(1).lin[0], TOL_BF16, label="27b b1")


def test_linear_batched_64():
    """64 sequences with their own trees and accepted paths."""
    check(workload_linear_27b(64, cfg=3).lin[0], TOL_BF16, label="27b b64")


def _custom(parents, paths, Hk, Hv, dk, dv, dtype, cfg=50):
    return gen_lin(cfg, parents, paths, Hk, Hv, dk, dv, dtype)


@pytest.mark.parametrize("dk,dv,dtype", [(16, 16, "bf16"), (32, 64, "bf16"), (64, 32, "f32"),
                                         (128, 16, "bf16"), (16, 128, "f32"), (128, 128, "f32")])
def test_head_sizes(dk, dv, dtype):
    parents, paths = trees_for(51, 2, "ddtree")
    L = _custom(parents, paths, 2, 4, dk, dv, dtype)
    check(L, TOL_BF16 if dtype == "bf16" else TOL_F32, label=f"dk{dk} dv{dv} {dtype}")


@pytest.mark.parametrize("n", [1, 2, 9, 17, 33, 64])
def test_tree_sizes_and_deep_chain(n):
    """Node counts across every tile configuration, including a 64-deep chain."""
    rng = np.random.default_rng(n)
    parents = [tree_chain(n), tree_ddtree(rng, budget=n, max_depth=12, topk=5)]
    paths = [np.arange(n, dtype=np.int32), random_root_leaf_path(rng, parents[1], len(parents[1]))]
    L = _custom(parents, paths, 2, 6, 64, 64, "bf16", cfg=60 + n)
    check(L, TOL_BF16, label=f"n{n}")


def test_ragged_batch_and_empty_path():
    """Sequences with different node counts; path_len 0 leaves that state unchanged."""
    rng = np.random.default_rng(5)
    parents = [tree_ddtree(rng, budget=22), tree_ddtree(rng, budget=5), np.array([-1], np.int32)]
    paths = [random_root_leaf_path(rng, p, len(p)) for p in parents]
    L = _custom(parents, paths, 4, 8, 128, 128, "bf16", cfg=70)
    L.path_len[1] = 0
    out, cap, st = check_no_path(L)
    np.testing.assert_array_equal(st[1], L.state[1])


def check_no_path(L):
    out, cap, st, _ = run_gpu(L)
    ro, rd, _ = run_oracle(L)
    mask = valid_rows(L.n_nodes, L.parent.shape[1])
    assert rel_err(out, ro, mask) <= TOL_BF16 and rel_err(cap, rd, mask) <= TOL_BF16
    for b in range(len(L.path_len)):
        if L.path_len[b] == 0:
            continue
        one = oracle.lin_commit_replay(L.state[b:b + 1], L.path[b:b + 1], L.path_len[b:b + 1], L.k[b:b + 1],
                                       L.v[b:b + 1], L.g[b:b + 1], L.beta[b:b + 1], L.parent[b:b + 1],
                                       L.n_nodes[b:b + 1], L.dtype)
        assert rel_err(st[b], one[0]) <= TOL_BF16
    return out, cap, st


def test_tiled_head_grouping():
    parents, paths = trees_for(52, 2, "ddtree")
    L = _custom(parents, paths, 4, 12, 64, 64, "bf16", cfg=52)
    check(L, TOL_BF16, head_group="tiled", label="tiled")


def test_commit_selects_exactly_the_path():
    """Every node gets a very different v, so a wrong node in the commit (or a wrong parent
    in verify) would move the state by O(1), far outside the tolerance."""
    parents, paths = trees_for(53, 4, "ddtree")
    L = _custom(parents, paths, 2, 4, 32, 32, "f32", cfg=53)
    L.v *= (1.0 + 10.0 * np.arange(L.v.shape[1]))[None, :, None, None].astype(np.float32)
    check(L, TOL_F32, label="distinct v")
    # every prefix of a path, and a path that stops at an interior node
    for Lp in range(1, int(L.path_len[0]) + 1):
        L2 = _custom(parents, paths, 2, 4, 32, 32, "f32", cfg=53)
        L2.v = L.v
        L2.path_len[:] = np.minimum(L2.path_len, Lp)
        check(L2, TOL_F32, label=f"prefix {Lp}")


def test_deterministic_and_batch_invariant():
    W = workload_linear_27b(4, cfg=3)
    L = W.lin[0]
    o1, c1, s1, _ = run_gpu(L)
    o2, c2, s2, _ = run_gpu(L)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(s1, s2)
    one = workload_linear_27b(1, cfg=3, seq_ids=[2]).lin[0]
    ob, cb, sb, _ = run_gpu(one)
    n = int(one.n_nodes[0])
    assert np.array_equal(ob[0, :n], o1[2, :n]) and np.array_equal(sb[0], s1[2])


def test_verify_does_not_touch_state():
    L = workload_linear_27b(2, cfg=3).lin[0]
    d = lin_to_device(L)
    before = d["state"].clone()
    tvl.lin_tree_verify(d["q"], d["k"], d["v"], d["g"], d["beta"], d["state"], d["parent"], d["n_nodes"], L.scale)
    torch.cuda.synchronize()
    assert torch.equal(before, d["state"])

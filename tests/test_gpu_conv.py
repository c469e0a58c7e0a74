"""Parity of the HIP tree-aware causal convolution and its window commit against the oracle.

Tolerance: the kernel sums K fp32 products (fused multiply-adds) of exactly converted
inputs, and SiLU runs in fp32: max |gpu - oracle| <= 1e-5 x RMS(oracle) per output.  The
commit copies inputs into the window, so it is compared bit for bit (bf16 -> fp32 is exact).
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import t_bits, t_f32, t_i32, rel_err, valid_rows
from workloads import (gen_conv, workload_conv, trees_for, tree_chain, tree_ddtree, random_root_leaf_path,
                       pad_trees)

pytestmark = pytest.mark.gpu

TOL = 1e-5


def to_dev(X):
    x = t_bits(X.x) if X.dtype == "bf16" else t_f32(X.x)
    return dict(x=x, w=t_f32(X.weight), st=t_f32(X.state), parent=t_i32(X.parent), n=t_i32(X.n_nodes),
                path=t_i32(X.path), plen=t_i32(X.path_len))


def check(X, activation="none", label=""):
    d = to_dev(X)
    B, N = X.parent.shape
    y = torch.full((B, N, X.C), float("nan"), device="cuda")
    tvl.conv_tree_verify(d["x"], d["w"], d["st"], d["parent"], d["n"], activation, y=y)
    st = d["st"].clone()
    tvl.conv_tree_commit(st, d["x"], d["path"], d["plen"])
    torch.cuda.synchronize()
    y, st = y.cpu().numpy(), st.cpu().numpy()
    ry = oracle.conv_tree_verify(X.x, X.dtype, X.weight, X.state, X.parent, X.n_nodes, activation)
    rs = oracle.conv_tree_commit(X.x, X.dtype, X.state, X.path, X.path_len)
    mask = valid_rows(X.n_nodes, N)
    e = rel_err(y, ry, mask)
    print(f"[conv {label}] K={X.K} C={X.C} {X.dtype} {activation}: y {e:.2e} x RMS; window bit-exact "
          f"{np.array_equal(st, rs.astype(np.float32))}")
    assert np.isnan(y[~mask]).all(), "padding rows were written"
    assert e <= TOL
    assert np.array_equal(st, rs.astype(np.float32))


def test_conv_batched_width():
    """64 sequences x 22-node trees, 10240 channels (q|k|v of the 27B-width linear layer), K = 4."""
    check(workload_conv(64), "none", "b64")


@pytest.mark.parametrize("activation", ["none", "silu"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_dtypes_and_activation(dtype, activation):
    parents, paths = trees_for(90, 3, "ddtree")
    check(gen_conv(90, parents, paths, 1024, 4, dtype), activation, f"{dtype}")


@pytest.mark.parametrize("K", [2, 3, 5, 8])
def test_conv_widths_deep_and_shallow(K):
    """Other widths; a chain deeper than the window, a root alone (all window rows from the
    committed state), a 64-node tree, paths of every length up to the window and beyond."""
    rng = np.random.default_rng(K)
    parents = [tree_chain(12), np.array([-1], np.int32), tree_ddtree(rng, budget=64, max_depth=16, topk=6),
               tree_ddtree(rng, budget=9)]
    parent, n = pad_trees(parents)
    paths = [np.arange(min(12, K + 1), dtype=np.int32), np.array([0], np.int32),
             random_root_leaf_path(rng, parent[2], int(n[2])), np.zeros(0, np.int32)]
    check(gen_conv(91, parents, paths, 520, K, "bf16"), "silu", f"K{K}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_conv_ragged_channel_chunk(dtype):
    """3080 channels: one full 2048-channel workgroup, then one whose first 1024 channels are
    all present and whose second half holds only 8 (a thread's two channel quads split)."""
    parents, paths = trees_for(92, 3, "ddtree")
    check(gen_conv(92, parents, paths, 3080, 4, dtype), "silu", f"C3080 {dtype}")


def test_conv_deterministic():
    X = workload_conv(4, C=2048)
    d = to_dev(X)
    y1 = tvl.conv_tree_verify(d["x"], d["w"], d["st"], d["parent"], d["n"])
    y2 = tvl.conv_tree_verify(d["x"], d["w"], d["st"], d["parent"], d["n"])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)

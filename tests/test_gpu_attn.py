"""Parity of the HIP tree attention against the fp64 oracle.

Tolerance: max |gpu - oracle| <= 2e-3 x RMS(oracle) for the outputs (bf16 queries, Q8_0 /
Q4_0 caches, fp32 outputs) and |lse error| <= 1e-3 (natural log).  K and V are dequantised
exactly (fp16 hi + lo) and the softmax weights P enter as an fp16 pair hi + lo, so the
kernel's error is fp32 accumulation order and exp2: measured a few 1e-6 x RMS.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import attn_to_device, rel_err, valid_rows
from workloads import (workload_attention_27b, workload_long_context, gen_attn, trees_for, tree_chain,
                       tree_ddtree, AttnInputs)

pytestmark = pytest.mark.gpu

TOL = 2e-3
TOL_LSE = 1e-3


def run_gpu(A, sentinel=True):
    d = attn_to_device(A)
    B, N = A.parent.shape
    out = torch.full((B, N, A.Hq, A.D), float("nan"), device="cuda") if sentinel else None
    lse = torch.full((B, N, A.Hq), float("nan"), device="cuda") if sentinel else None
    out, lse = tvl.attn_tree_verify(d["q"], d["k_cache"], d["v_cache"], A.k_type, A.v_type, d["n_past"],
                                    d["parent"], d["n_nodes"], A.window, A.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(A, label=""):
    out, lse = run_gpu(A)
    ro, rl = oracle.attn_tree_verify(A.q, A.k_cache, A.v_cache, A.k_type, A.v_type, A.n_past, A.parent,
                                     A.n_nodes, A.window, A.scale, A.Hkv)
    mask = valid_rows(A.n_nodes, A.parent.shape[1])
    e = rel_err(out, ro, mask)
    el = float(np.max(np.abs(lse[mask] - rl[mask])))
    print(f"[attn {label}] out {e:.2e} x RMS, lse {el:.2e}")
    assert np.isnan(out[~mask]).all() and np.isnan(lse[~mask]).all(), "padding rows were written"
    assert e <= TOL and el <= TOL_LSE
    return out, lse


def test_attention_27b_window():
    """24 query / 4 KV heads, D=256, 4096 committed Q8_0 slots, window 2048, 22-node tree."""
    check(workload_attention_27b(1).attn[0], "27b w2048")


def test_attention_27b_full():
    check(workload_attention_27b(1, window=0).attn[0], "27b w0")


@pytest.mark.parametrize("kt,vt", [("q4_0", "q4_0"), ("q8_0", "q4_0"), ("q4_0", "q8_0")])
def test_kv_type_pairs(kt, vt):
    parents, _ = trees_for(80, 2, "ddtree")
    A = gen_attn(80, parents, 24, 4, 256, 700, kt, vt, 300)
    check(A, f"{kt}/{vt}")


def test_batched_64():
    """64 sequences, each with its own 22-node tree, T=4096, Q8_0, window 2048."""
    from workloads import workload_batched
    check(workload_batched(64).attn[0], "b64")


@pytest.mark.parametrize("T,window", [(0, 0), (0, 5), (37, 1), (37, 0), (100, 3), (1000, 64)])
def test_edges(T, window):
    """No history, a window of one (each node sees only itself), tiny windows, ragged tails."""
    rng = np.random.default_rng(T * 7 + window)
    parents = [tree_ddtree(rng, budget=22), tree_chain(9), np.array([-1], np.int32)]
    A = gen_attn(81, parents, 24, 4, 256, T, "q8_0", "q8_0", window)
    check(A, f"T{T} w{window}")


def test_ragged_history_and_other_grouping():
    """Different n_past per sequence; 2 query heads per KV head; 64-node tree."""
    rng = np.random.default_rng(9)
    parents = [tree_ddtree(rng, budget=64, max_depth=16, topk=6), tree_chain(40), tree_ddtree(rng, budget=5)]
    A = gen_attn(82, parents, 8, 4, 256, [513, 70, 1999], "q8_0", "q4_0", 256, tcap=2100)
    check(A, "ragged")


@pytest.mark.parametrize("nodes", [64, 50])
def test_many_row_blocks(nodes):
    """Trees whose rows (nodes x 6 query heads) need three row blocks: 384 rows as 8 + 8 + 8
    row tiles, 300 rows as 7 + 7 + 5; every row against the oracle, window 0 and a short
    window."""
    rng = np.random.default_rng(11 + nodes)
    parents = [tree_ddtree(rng, budget=nodes, max_depth=20, topk=6), tree_chain(nodes)]
    for window in (0, 37):
        A = gen_attn(83, parents, 24, 4, 256, [300, 129], "q8_0", "q4_0", window)
        check(A, f"{nodes} nodes w{window}")


@pytest.mark.parametrize("window", [0, 2048])
def test_long_context_all_rows(window):
    """131072 committed Q4_0 slots (K and V), window 0 and 2048: every row of the layer (22
    nodes x 24 query heads) against the oracle's dense masked softmax."""
    W = workload_long_context(window=window, n_lin=0, n_attn=1)
    A = W.attn[0]
    out, lse = run_gpu(A)
    ro, rl = oracle.attn_tree_verify_dense(A.q, A.k_cache, A.v_cache, A.k_type, A.v_type, A.n_past, A.parent,
                                           A.n_nodes, A.window, A.scale, A.Hkv)
    mask = valid_rows(A.n_nodes, A.parent.shape[1])
    e = rel_err(out, ro, mask)
    el = float(np.max(np.abs(lse[mask] - rl[mask])))
    print(f"[attn long w{window}] all {int(mask.sum()) * A.Hq} rows: out {e:.2e} x RMS, lse {el:.2e}")
    assert e <= TOL and el <= TOL_LSE
    assert np.isnan(out[~mask]).all()


def test_deterministic_and_batch_invariant():
    from workloads import workload_batched
    A = workload_batched(3).attn[0]
    o1, l1 = run_gpu(A)
    o2, l2 = run_gpu(A)
    assert np.array_equal(o1, o2, equal_nan=True)
    one = workload_batched(1, seq_ids=[1]).attn[0]
    ob, lb = run_gpu(one)
    n = int(one.n_nodes[0])
    # The KV split plan depends on the batch size, so the two runs accumulate in different
    # orders; both are fp32 sums of the same exactly formed terms, so they agree to a few
    # fp32 rounding steps, far inside the parity tolerance.
    e = rel_err(ob[0, :n], o1[1, :n])
    el = float(np.max(np.abs(lb[0, :n] - l1[1, :n])))
    print(f"[attn batch invariance] out {e:.2e} x RMS, lse {el:.2e}")
    assert e <= 1e-5 and el <= 1e-5


def _scaled_queries(A, factor_rows):
    """A copy of A whose query rows (node, head) are multiplied by powers of two (exact in
    bf16): factor_rows maps node -> factor."""
    import dataclasses
    from workloads import f32_to_bf16_bits
    from oracle.delta import bf16_bits_to_f64
    q = bf16_bits_to_f64(A.q)
    for node, f in factor_rows.items():
        q[:, node] *= f
    return dataclasses.replace(A, q=f32_to_bf16_bits(q.astype(np.float32)))


def test_query_range_beyond_fp16():
    """Queries far outside fp16's range.  Each query row enters the matrix cores pre-scaled by
    a power of two, so (1) every query times 2^20 with the scale times 2^-20, and (2) times
    2^-30 with the scale times 2^30, give the unscaled call's outputs bit for bit; (3) single
    nodes whose queries reach 10^5 .. 10^6 (beyond fp16's 65504) or 10^-9 match the oracle."""
    import dataclasses
    rng = np.random.default_rng(5)
    parents = [tree_ddtree(rng, budget=22), tree_chain(7)]
    A = gen_attn(83, parents, 24, 4, 256, [300, 120], "q8_0", "q4_0", 0)
    o0, l0 = run_gpu(A)
    for f in (2.0 ** 20, 2.0 ** -30):
        Af = dataclasses.replace(_scaled_queries(A, {i: f for i in range(A.parent.shape[1])}), scale=A.scale / f)
        of, lf = run_gpu(Af)
        assert np.array_equal(of, o0, equal_nan=True) and np.array_equal(lf, l0, equal_nan=True), f
    Am = _scaled_queries(A, {1: 2.0 ** 17, 3: 2.0 ** 18, 5: 2.0 ** -30})
    out, lse = run_gpu(Am)
    assert np.abs(bf16_max(Am.q)) > 65504.0
    ro, rl = oracle.attn_tree_verify(Am.q, Am.k_cache, Am.v_cache, Am.k_type, Am.v_type, Am.n_past, Am.parent,
                                     Am.n_nodes, Am.window, Am.scale, Am.Hkv)
    mask = valid_rows(Am.n_nodes, Am.parent.shape[1])
    e = rel_err(out, ro, mask)
    el = float(np.max(np.abs(lse[mask] - rl[mask]) / np.maximum(1.0, np.abs(rl[mask]))))
    print(f"[attn large queries] out {e:.2e} x RMS, lse rel {el:.2e}")
    assert e <= TOL and el <= TOL_LSE


def bf16_max(q):
    from oracle.delta import bf16_bits_to_f64
    return np.abs(bf16_bits_to_f64(q)).max()

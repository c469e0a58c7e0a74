"""The second workload: draft budgets 8, 16 and 40 and asymmetric K/V cache types, on the
same kernels ("Luce DFlash" README: the budget-22 default, budget 40 on the larger card,
budgets 8 and 16 in the sweeps; "Asymmetric K/V quantization": per-side cache types).

Budget 8 is a pure chain; budget 40 takes the linear verify's 33-64-node variant and two
row blocks of attention per KV head.  Tolerances as in the main parity tests.
"""
import numpy as np
import pytest

import oracle
from test_gpu_attn import TOL, TOL_LSE, check as attn_check, run_gpu as attn_run
from test_gpu_lin import TOL_BF16, check as lin_check, run_gpu as lin_run
from tvutil import rel_err
from workloads import workload_batched

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("budget", [8, 16, 40])
def test_linear_budgets(budget):
    lin_check(workload_batched(4, budget=budget).lin[0], TOL_BF16, label=f"budget {budget}")


@pytest.mark.parametrize("budget", [8, 16, 40])
@pytest.mark.parametrize("kt,vt", [("q8_0", "q4_0"), ("q4_0", "q8_0")])
def test_attention_budgets_asymmetric(budget, kt, vt):
    attn_check(workload_batched(2, budget=budget, k_type=kt, v_type=vt).attn[0], f"budget {budget} {kt}/{vt}")


def test_budget40_batched_full():
    """64 sequences x 40-node trees, Q8_0 K + Q4_0 V, at the benchmark's own shape: every
    attention row of every sequence, and the linear outputs, deltas and committed states of
    all 64 sequences, against the oracle."""
    W = workload_batched(64, budget=40, k_type="q8_0", v_type="q4_0")
    A, L = W.attn[0], W.lin[0]
    out, lse = attn_run(A)
    ro, rl = oracle.attn_tree_verify(A.q, A.k_cache, A.v_cache, A.k_type, A.v_type, A.n_past, A.parent, A.n_nodes,
                                     A.window, A.scale, A.Hkv)
    mask = np.arange(A.q.shape[1])[None, :] < np.asarray(A.n_nodes)[:, None]
    e, el = rel_err(out[mask], ro[mask]), float(np.max(np.abs(lse[mask] - rl[mask])))
    print(f"[budget 40 b64] attention, all {int(mask.sum()) * A.Hq} rows: {e:.2e} x RMS, lse {el:.2e}")
    assert e <= TOL and el <= TOL_LSE

    o, cap, st, _ = lin_run(L)
    ro, rd = oracle.lin_tree_verify(L.q, L.k, L.v, L.g, L.beta, L.state, L.parent, L.n_nodes, L.scale, L.dtype)
    rs = oracle.lin_commit_replay(L.state, L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes, L.dtype)
    lm = np.arange(L.parent.shape[1])[None, :] < np.asarray(L.n_nodes)[:, None]
    eo, ed, es = rel_err(o[lm], ro[lm]), rel_err(cap[lm], rd[lm]), rel_err(st, rs)
    print(f"[budget 40 b64] linear, all 64 sequences: out {eo:.2e} delta {ed:.2e} state {es:.2e}")
    assert eo <= TOL_BF16 and ed <= TOL_BF16 and es <= TOL_BF16

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


def test_budget40_batched_sampled():
    """64 sequences x 40-node trees, Q8_0 K + Q4_0 V: sampled attention rows of every
    sequence, and whole linear outputs of three sequences, against the oracle."""
    W = workload_batched(64, budget=40, k_type="q8_0", v_type="q4_0")
    A, L = W.attn[0], W.lin[0]
    out, lse = attn_run(A)
    rng = np.random.default_rng(40)
    rows = [(b, int(rng.integers(0, int(A.n_nodes[b]))), int(rng.integers(0, A.Hq))) for b in range(64)]
    rows += [(5, int(A.n_nodes[5]) - 1, A.Hq - 1), (63, 0, 0)]
    ro, rl = oracle.attn_tree_verify_rows(A.q, A.k_cache, A.v_cache, A.k_type, A.v_type, A.n_past, A.parent,
                                          A.n_nodes, A.window, A.scale, A.Hkv, rows)
    got = np.stack([out[b, i, h] for b, i, h in rows])
    gl = np.array([lse[b, i, h] for b, i, h in rows])
    e, el = rel_err(got, ro), float(np.max(np.abs(gl - rl)))
    print(f"[budget 40 b64] attention sampled {e:.2e} x RMS, lse {el:.2e}")
    assert e <= TOL and el <= TOL_LSE

    o, cap, st, _ = lin_run(L)
    for b in (0, 31, 63):
        sl = slice(b, b + 1)
        ro, rd = oracle.lin_tree_verify(L.q[sl], L.k[sl], L.v[sl], L.g[sl], L.beta[sl], L.state[sl], L.parent[sl],
                                        L.n_nodes[sl], L.scale, L.dtype)
        rs = oracle.lin_commit_replay(L.state[sl], L.path[sl], L.path_len[sl], L.k[sl], L.v[sl], L.g[sl],
                                      L.beta[sl], L.parent[sl], L.n_nodes[sl], L.dtype)
        n = int(L.n_nodes[b])
        eo, ed, es = rel_err(o[b, :n], ro[0, :n]), rel_err(cap[b, :n], rd[0, :n]), rel_err(st[b], rs[0])
        print(f"[budget 40 b64] linear seq {b}: out {eo:.2e} delta {ed:.2e} state {es:.2e}")
        assert eo <= TOL_BF16 and ed <= TOL_BF16 and es <= TOL_BF16

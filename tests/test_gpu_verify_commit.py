"""Parity of the fused commit + verify (lin_tree_verify_commit) against the oracle.

The previous step's accepted path is committed into the state (from its k, g and captured
deltas) inside this step's verify.  Compared with oracle.lin_tree_verify_commit (the commit
replayed from v and beta, then the plain verify from the stored fp32 state) and with the
unfused calls.  Tolerances as for the separate calls: 2e-3 x RMS (bf16 inputs), 1e-4 x RMS
(fp32 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import lin_to_device, rel_err, valid_rows
from workloads import gen_lin, trees_for, tree_chain, tree_ddtree, random_root_leaf_path

pytestmark = pytest.mark.gpu


def two_steps(Hk, Hv, dk, dv, dtype, B=3, budgets=(22, 22), cfg=120, empty=()):
    p1, a1 = trees_for(cfg, B, "ddtree", budget=budgets[0]) if budgets[0] != 22 else trees_for(cfg, B, "ddtree")
    p2, a2 = trees_for(cfg + 1, B, "ddtree", budget=budgets[1]) if budgets[1] != 22 else trees_for(cfg + 1, B, "ddtree")
    a1 = [np.zeros(0, np.int32) if b in empty else a for b, a in enumerate(a1)]
    L1 = gen_lin(cfg, p1, a1, Hk, Hv, dk, dv, dtype)
    L2 = gen_lin(cfg + 1, p2, a2, Hk, Hv, dk, dv, dtype)
    return L1, L2


def check(L1, L2, tol, label=""):
    d1, d2 = lin_to_device(L1), lin_to_device(L2)
    state = d1["state"].clone()
    _, cap1 = tvl.lin_tree_verify(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], state, d1["parent"],
                                  d1["n_nodes"], L1.scale)
    B, N = L2.parent.shape
    out = torch.full((B, N, L2.Hv, L2.dv), float("nan"), device="cuda")
    cap = torch.full_like(out, float("nan"))
    tvl.lin_tree_verify_commit(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], state, d2["parent"], d2["n_nodes"],
                               L2.scale, d1["path"], d1["path_len"], d1["k"], d1["g"], cap1, out=out, cap_delta=cap)
    # the unfused calls on a copy of the original state
    st_u = d1["state"].clone()
    tvl.lin_tree_commit(st_u, d1["path"], d1["path_len"], d1["k"], d1["g"], cap1)
    out_u, cap_u = tvl.lin_tree_verify(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], st_u, d2["parent"],
                                       d2["n_nodes"], L2.scale)
    torch.cuda.synchronize()
    prev = (L1.path, L1.path_len, L1.k, L1.v, L1.g, L1.beta, L1.parent, L1.n_nodes)
    rs, ro, rd = oracle.lin_tree_verify_commit(L1.state, prev, L2.q, L2.k, L2.v, L2.g, L2.beta, L2.parent,
                                               L2.n_nodes, L2.scale, L2.dtype)
    mask = valid_rows(L2.n_nodes, N)
    o, c, s = out.cpu().numpy(), cap.cpu().numpy(), state.cpu().numpy()
    e_o, e_d, e_s = rel_err(o, ro, mask), rel_err(c, rd, mask), rel_err(s, rs)
    e_fu = max(rel_err(o, out_u.cpu().numpy(), mask), rel_err(s, st_u.cpu().numpy()))
    print(f"[verify+commit {label}] out {e_o:.2e} delta {e_d:.2e} state {e_s:.2e}; vs unfused {e_fu:.2e}")
    assert np.isnan(o[~mask]).all(), "padding rows were written"
    assert e_o <= tol and e_d <= tol and e_s <= tol and e_fu <= tol
    return s


def test_fused_27b_width():
    """16 key / 48 value heads of 128, bf16, 22-node trees in both steps."""
    check(*two_steps(16, 48, 128, 128, "bf16"), 2e-3, "27b")


def _units_are_64_wide(B, Hv, dv):
    """The launcher narrows units below 64 channels only while a launch would give fewer than
    two units per compute unit; this returns whether this shape keeps 64-channel units."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return B * Hv * (dv // 64) >= 2 * cus


def test_fused_64_channel_units():
    """27B width with enough sequences that the launcher keeps 64-channel units (the width the
    batched step runs): every sequence of two steps compared with the oracle."""
    B = 8
    assert _units_are_64_wide(B, 48, 128), "this shape no longer exercises 64-channel units"
    L1, L2 = two_steps(16, 48, 128, 128, "bf16", B=B, cfg=160)
    check(L1, L2, 2e-3, "27b B8 cw64")


def test_fused_batched_step_shape():
    """The batched step itself: 64 sequences, 22-node trees, two steps through the fused call.
    Every sequence is compared with the oracle and with the separate calls."""
    B = 64
    assert _units_are_64_wide(B, 48, 128)
    # the batched step's linear layer (its trees and paths), and a second step of the same sequences
    L1, L2 = (gen_lin(c, *trees_for(c, B, "ddtree"), 16, 48, 128, 128, "bf16") for c in (3, 203))
    d1, d2 = lin_to_device(L1), lin_to_device(L2)
    state = d1["state"].clone()
    _, cap1 = tvl.lin_tree_verify(d1["q"], d1["k"], d1["v"], d1["g"], d1["beta"], state, d1["parent"],
                                  d1["n_nodes"], L1.scale)
    N = L2.parent.shape[1]
    out = torch.full((B, N, L2.Hv, L2.dv), float("nan"), device="cuda")
    cap = torch.full_like(out, float("nan"))
    tvl.lin_tree_verify_commit(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], state, d2["parent"], d2["n_nodes"],
                               L2.scale, d1["path"], d1["path_len"], d1["k"], d1["g"], cap1, out=out, cap_delta=cap)
    st_u = d1["state"].clone()
    tvl.lin_tree_commit(st_u, d1["path"], d1["path_len"], d1["k"], d1["g"], cap1)
    out_u, cap_u = tvl.lin_tree_verify(d2["q"], d2["k"], d2["v"], d2["g"], d2["beta"], st_u, d2["parent"],
                                       d2["n_nodes"], L2.scale)
    torch.cuda.synchronize()
    mask = valid_rows(L2.n_nodes, N)
    o, c, s = out.cpu().numpy(), cap.cpu().numpy(), state.cpu().numpy()
    e_fu = max(rel_err(o, out_u.cpu().numpy(), mask), rel_err(c, cap_u.cpu().numpy(), mask),
               rel_err(s, st_u.cpu().numpy()))
    assert np.isnan(o[~mask]).all(), "padding rows were written"
    prev = (L1.path, L1.path_len, L1.k, L1.v, L1.g, L1.beta, L1.parent, L1.n_nodes)
    rs, ro, rd = oracle.lin_tree_verify_commit(L1.state, prev, L2.q, L2.k, L2.v, L2.g, L2.beta, L2.parent,
                                               L2.n_nodes, L2.scale, L2.dtype)
    e_o, e_d, e_s = rel_err(o, ro, mask), rel_err(c, rd, mask), rel_err(s, rs)
    print(f"[verify+commit b64] out {e_o:.2e} delta {e_d:.2e} state {e_s:.2e}; vs unfused {e_fu:.2e} (all 64)")
    assert e_o <= 2e-3 and e_d <= 2e-3 and e_s <= 2e-3 and e_fu <= 2e-3


def test_fused_tree_sizes_differ_and_empty_paths():
    """Previous step 40 nodes (the wide kernel's tree size), this step 8 (a chain); one
    sequence accepted nothing in the previous step: its state stays bit-identical."""
    L1, L2 = two_steps(4, 12, 128, 128, "bf16", B=3, budgets=(40, 8), empty=(1,))
    s = check(L1, L2, 2e-3, "40 -> 8")
    assert np.array_equal(s[1], L1.state[1]), "a sequence with nothing accepted had its state changed"
    L1, L2 = two_steps(4, 12, 128, 128, "bf16", B=2, budgets=(8, 40), cfg=130)
    check(L1, L2, 2e-3, "8 -> 40")


def test_fused_wide_trees_f32():
    """fp32 inputs with 40-node trees in both steps: the fused call runs in the wide kernel's
    fp32 instantiation (k/q operands in registers, one wave per SIMD)."""
    check(*two_steps(2, 4, 128, 128, "f32", B=2, budgets=(40, 40), cfg=170), 1e-4, "40 -> 40 f32")


@pytest.mark.parametrize("dk,dv,dtype", [(16, 16, "f32"), (32, 64, "bf16"), (64, 32, "f32"), (128, 128, "f32")])
def test_fused_head_sizes(dk, dv, dtype):
    check(*two_steps(2, 4, dk, dv, dtype, B=2, cfg=140 + dk + dv), 1e-4 if dtype == "f32" else 2e-3, f"{dk}/{dv} {dtype}")


def test_fused_deep_chain_path():
    """A previous path longer than one staging chunk (four entries): a 20-node chain
    accepted to its end."""
    B = 2
    p1 = [tree_chain(20), tree_chain(20)]
    a1 = [np.arange(20, dtype=np.int32), np.arange(7, dtype=np.int32)]
    rng = np.random.default_rng(3)
    p2 = [tree_ddtree(rng, budget=22), tree_ddtree(rng, budget=22)]
    a2 = [random_root_leaf_path(rng, p, len(p)) for p in p2]
    L1 = gen_lin(150, p1, a1, 4, 8, 128, 128, "bf16")
    L2 = gen_lin(151, p2, a2, 4, 8, 128, 128, "bf16")
    check(L1, L2, 2e-3, "deep chain")

"""Parity of the pending bank (lin_tree_verify_bank, lin_bank_flush) against the oracle.

Several steps run through the bank.  Each verify starts from the committed state -- the
stored state, the bank's entries and the previous step's accepted path -- and then either
appends that path to the bank or, when it does not fit (E + L > Emax) or a flush is asked
for, stores the committed state and empties the bank.  Every step's outputs and deltas are
compared with oracle.lin_tree_verify_bank, whose pending list holds every earlier step (the
values do not depend on when the bank is flushed).  Where a flush is due the stored state is
compared with the oracle's committed state; elsewhere it must be unchanged bit for bit.
Tolerances: 2e-3 x RMS (bf16 inputs), 1e-4 x RMS (fp32 inputs), as for the other linear calls.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import lin_to_device, rel_err, valid_rows
from workloads import gen_lin, trees_for, tree_chain

pytestmark = pytest.mark.gpu


def _prev(L):
    return (L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes)


def _slice(L, idx):
    import dataclasses
    idx = np.asarray(idx)
    return dataclasses.replace(L, q=L.q[idx], k=L.k[idx], v=L.v[idx], g=L.g[idx], beta=L.beta[idx],
                               state=L.state[idx], parent=L.parent[idx], n_nodes=L.n_nodes[idx],
                               path=L.path[idx], path_len=L.path_len[idx])


def _committed(S0, steps, head_group):
    """The oracle's committed state after every step in ``steps``: one commit per step."""
    S = np.asarray(S0, np.float32).astype(np.float64)
    for s in steps:
        S = oracle.lin_commit_replay(S, s.path, s.path_len, s.k, s.v, s.g, s.beta, s.parent, s.n_nodes, s.dtype,
                                     head_group).astype(np.float32).astype(np.float64)
    return S


def run_bank(steps, Emax, tol, force=(), check_seqs=None, head_group="contiguous", label=""):
    """Runs ``steps`` (LinInputs with their accepted paths) through the bank from the first
    step's state, then flushes.  ``force``: steps whose verify is asked to flush.
    ``check_seqs``: the sequences compared with the oracle (all if None).  Returns the list
    of per-step flush masks."""
    L0 = steps[0]
    B, Hk, Hv, dk, dv = L0.q.shape[0], L0.Hk, L0.Hv, L0.dk, L0.dv
    ddt = torch.bfloat16 if L0.dtype == "bf16" else torch.float32
    dev_steps = [lin_to_device(L) for L in steps]
    state = dev_steps[0]["state"].clone()
    bank = tvl.lin_bank_empty(B, Hk, Hv, dk, dv, Emax, ddt, "cuda")
    E = np.zeros(B, np.int64)                        # the bank length the header's rule predicts
    seqs = list(range(B)) if check_seqs is None else list(check_seqs)
    flush_log = []
    prev = None
    for t, L in enumerate(steps):
        d = dev_steps[t]
        N = L.parent.shape[1]
        if prev is None:                             # nothing pending before the first step
            p = (d["path"], torch.zeros_like(d["path_len"]), d["k"], d["g"],
                 torch.zeros((B, N, Hv, dv), dtype=torch.float32, device="cuda"))
            Lp = np.zeros(B, np.int64)
        else:
            p = prev
            Lp = steps[t - 1].path_len.astype(np.int64)
        before = state.cpu().numpy()
        flush = t in force
        out = torch.full((B, N, Hv, dv), float("nan"), device="cuda")
        out, cap = tvl.lin_tree_verify_bank(d["q"], d["k"], d["v"], d["g"], d["beta"], state, d["parent"],
                                            d["n_nodes"], L.scale, *p, bank, flush=flush, head_group=head_group,
                                            out=out)
        torch.cuda.synchronize()
        flushed = flush | (Lp > Emax - E)
        written = flushed & (E + Lp > 0)
        flush_log.append(flushed)
        after = state.cpu().numpy()
        assert np.array_equal(after[~written], before[~written]), f"step {t}: a state without a flush was written"
        E = np.where(flushed, 0, E + Lp)
        assert np.array_equal(bank.length.cpu().numpy(), E), f"step {t}: bank lengths"
        # oracle: every earlier step pending, from the first state
        A = [_slice(x, seqs) for x in steps[:t + 1]]
        rs, ro, rd = oracle.lin_tree_verify_bank(A[0].state, [_prev(x) for x in A[:t]], A[t].q, A[t].k, A[t].v,
                                                 A[t].g, A[t].beta, A[t].parent, A[t].n_nodes, A[t].scale, A[t].dtype,
                                                 head_group)
        mask = valid_rows(A[t].n_nodes, N)
        o, c = out.cpu().numpy()[seqs], cap.cpu().numpy()[seqs]
        e_o, e_d = rel_err(o, ro, mask), rel_err(c, rd, mask)
        w = written[seqs]
        e_s = rel_err(after[seqs][w], rs[w]) if w.any() else 0.0
        print(f"[bank {label} step {t}] out {e_o:.2e} delta {e_d:.2e} stored {int(w.sum())} state {e_s:.2e} "
              f"E {E.min()}..{E.max()}")
        assert np.isnan(o[~mask]).all(), "padding rows were written"
        assert e_o <= tol and e_d <= tol and e_s <= tol
        prev = (d["path"], d["path_len"], d["k"], d["g"], cap)
    # the final flush: the stored state is every step committed
    tvl.lin_bank_flush(state, *prev, bank, head_group=head_group)
    torch.cuda.synchronize()
    assert (bank.length.cpu().numpy() == 0).all()
    ref = _committed(_slice(steps[0], seqs).state, [_slice(x, seqs) for x in steps], head_group)
    e_f = rel_err(state.cpu().numpy()[seqs], ref)
    print(f"[bank {label} final flush] state {e_f:.2e}")
    assert e_f <= tol
    return flush_log


def ddtree_steps(cfg, B, Hk, Hv, dk, dv, dtype, T, budget=22):
    return [gen_lin(cfg + t, *trees_for(cfg + t, B, "ddtree", budget=budget), Hk, Hv, dk, dv, dtype)
            for t in range(T)]


def test_bank_steps_27b_width():
    """16/48 heads of 128 at a small batch, bf16, 22-node trees, twelve steps through a
    32-entry bank: it fills and is flushed on its own."""
    steps = ddtree_steps(300, 3, 16, 48, 128, 128, "bf16", 12)
    log = run_bank(steps, 32, 2e-3, label="27b")
    assert sum(int(f.sum()) for f in log) > 0, "the bank never filled: the steps no longer exercise a flush"


def test_bank_fills_exactly_and_forced_flush():
    """Chains of 16 accepted to their end: the bank holds 16, 32, 48 and then exactly 64 = Emax
    entries (two full matrix steps) before a forced flush; the other sequence accepts fewer."""
    B = 2
    steps = [gen_lin(320 + t, [tree_chain(16)] * B, [np.arange(16 if b == 0 else 5 + t, dtype=np.int32)
                                                    for b in range(B)], 4, 8, 128, 128, "bf16")
             for t in range(7)]
    log = run_bank(steps, 64, 2e-3, force=(5,), label="64 entries")
    assert not log[4][0] and log[5][0]


def test_bank_flushes_when_the_path_does_not_fit():
    """12 of 12 accepted each step into a 32-entry bank: 12, 24, then the third path does not
    fit and the verify stores the committed state instead; then the bank refills."""
    B = 2
    steps = [gen_lin(380 + t, [tree_chain(12)] * B, [np.arange(12, dtype=np.int32), np.arange(2, dtype=np.int32)],
                     2, 4, 64, 64, "bf16") for t in range(6)]
    log = run_bank(steps, 32, 2e-3, label="fill")
    assert [bool(f[0]) for f in log] == [False, False, False, True, False, False]
    assert not any(bool(f[1]) for f in log)


@pytest.mark.parametrize("dk,dv,dtype", [(16, 16, "f32"), (32, 64, "bf16"), (64, 32, "f32"), (128, 128, "f32")])
def test_bank_head_sizes(dk, dv, dtype):
    steps = ddtree_steps(340 + dk + dv, 2, 2, 4, dk, dv, dtype, 6)
    run_bank(steps, 32, 1e-4 if dtype == "f32" else 2e-3, label=f"{dk}/{dv} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bank_decays_near_one(dtype):
    """Decays in [0.95, 1): earlier entries keep almost their whole weight, so the committed
    state is the sum of many terms of the size of the latest path's.  Ten steps of 128/128
    heads through a 32-entry bank (it fills and flushes); the stored state must meet the
    step's tolerance, which a c*delta rounded to two bf16 terms (2^-17 relative) would not
    for fp32 inputs."""
    import dataclasses
    rng = np.random.default_rng(17)
    steps = []
    for L in ddtree_steps(420, 2, 2, 4, 128, 128, dtype, 10):
        g = rng.uniform(0.95, 1.0, size=L.g.shape).astype(np.float32)
        if dtype == "bf16":
            g = (g.view(np.uint32) >> 16).astype(np.uint16)
        steps.append(dataclasses.replace(L, g=g))
    log = run_bank(steps, 32, 1e-4 if dtype == "f32" else 2e-3, label=f"decays near 1 {dtype}")
    assert sum(int(f.sum()) for f in log) > 0


def test_bank_tiled_heads_and_wide_trees():
    """Tiled head grouping, and 40-node trees (the wide verify kernel)."""
    steps = ddtree_steps(360, 2, 4, 12, 128, 128, "bf16", 5, budget=40)
    run_bank(steps, 32, 2e-3, head_group="tiled", label="tiled 40")


def test_bank_wide_trees_f32():
    """fp32 inputs with 40-node trees: the wide kernel's fp32 bank instantiation."""
    steps = ddtree_steps(365, 2, 2, 4, 128, 128, "f32", 4, budget=40)
    run_bank(steps, 32, 1e-4, label="40 f32")


def test_bank_batched_step_shape():
    """The batched step: 64 sequences, 22-node trees, 16/48 heads of 128, bf16; five steps
    through a 32-entry bank and a final flush, every sequence compared with the oracle (and
    with the separate calls in the next test)."""
    B = 64
    steps = [gen_lin(c, *trees_for(c, B, "ddtree"), 16, 48, 128, 128, "bf16") for c in (3, 203, 204, 205, 206)]
    run_bank(steps, 32, 2e-3, label="b64")


def test_bank_matches_separate_calls_all_sequences():
    """All 64 sequences of the batched shape: five banked steps (verify outputs and deltas)
    and the final flush against the separate verify and commit calls."""
    B = 64
    steps = [gen_lin(c, *trees_for(c, B, "ddtree"), 16, 48, 128, 128, "bf16") for c in (3, 203, 204, 205, 206)]
    d = [lin_to_device(L) for L in steps]
    state = d[0]["state"].clone()
    bank = tvl.lin_bank_empty(B, 16, 48, 128, 128, 32, torch.bfloat16, "cuda")
    st_u = d[0]["state"].clone()
    cap_b = cap_u = None
    for t, L in enumerate(steps):
        if t == 0:
            p = (d[0]["path"], torch.zeros_like(d[0]["path_len"]), d[0]["k"], d[0]["g"],
                 torch.zeros((B, L.parent.shape[1], 48, 128), device="cuda"))
        else:
            p = (d[t - 1]["path"], d[t - 1]["path_len"], d[t - 1]["k"], d[t - 1]["g"], cap_b)
            tvl.lin_tree_commit(st_u, d[t - 1]["path"], d[t - 1]["path_len"], d[t - 1]["k"], d[t - 1]["g"], cap_u)
        out, cap_b = tvl.lin_tree_verify_bank(d[t]["q"], d[t]["k"], d[t]["v"], d[t]["g"], d[t]["beta"], state,
                                              d[t]["parent"], d[t]["n_nodes"], L.scale, *p, bank)
        out_u, cap_u = tvl.lin_tree_verify(d[t]["q"], d[t]["k"], d[t]["v"], d[t]["g"], d[t]["beta"], st_u,
                                           d[t]["parent"], d[t]["n_nodes"], L.scale)
        torch.cuda.synchronize()
        mask = valid_rows(L.n_nodes, L.parent.shape[1])
        e_o = rel_err(out.cpu().numpy(), out_u.cpu().numpy(), mask)
        e_d = rel_err(cap_b.cpu().numpy(), cap_u.cpu().numpy(), mask)
        print(f"[bank vs separate, step {t}] out {e_o:.2e} delta {e_d:.2e}")
        assert e_o <= 2e-3 and e_d <= 2e-3
    tvl.lin_bank_flush(state, d[-1]["path"], d[-1]["path_len"], d[-1]["k"], d[-1]["g"], cap_b, bank)
    tvl.lin_tree_commit(st_u, d[-1]["path"], d[-1]["path_len"], d[-1]["k"], d[-1]["g"], cap_u)
    torch.cuda.synchronize()
    e_s = rel_err(state.cpu().numpy(), st_u.cpu().numpy())
    print(f"[bank vs separate] flushed state {e_s:.2e}")
    assert e_s <= 2e-3
    assert (bank.length.cpu().numpy() == 0).all()


def test_bank_flush_of_nothing_keeps_the_state():
    """An empty bank and an empty previous path: the flush leaves the state bit for bit."""
    L = gen_lin(390, *trees_for(390, 2, "ddtree"), 2, 4, 64, 64, "bf16")
    d = lin_to_device(L)
    state = d["state"].clone()
    bank = tvl.lin_bank_empty(2, 2, 4, 64, 64, 32, torch.bfloat16, "cuda")
    cap = torch.zeros((2, L.parent.shape[1], 4, 64), device="cuda")
    tvl.lin_bank_flush(state, d["path"], torch.zeros_like(d["path_len"]), d["k"], d["g"], cap, bank)
    torch.cuda.synchronize()
    assert np.array_equal(state.cpu().numpy(), L.state)

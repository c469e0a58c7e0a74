"""Pins for the linear-attention oracle (CPU only).

Each test checks the oracle against something other than itself: a hand-worked
example, a closed form of the delta rule, an independent matrix formulation of the
recurrence, or a brute-force re-run over each node's root path.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import lin_tree_verify, lin_commit_replay, lin_chain_recurrence, root_path
from oracle.delta import bf16_bits_to_f64
from workloads import (tree_small, tree_ddtree, tree_chain, random_root_leaf_path, rng_for,
                       gen_lin, trees_for, f32_to_bf16_bits, pad_trees, pad_paths)


def _handworked(golden_dir):
    with open(os.path.join(golden_dir, "delta_handworked.json")) as f:
        return json.load(f)


def _single(gj):
    """Pack the hand-worked tree as a B=1, one-head f32 problem."""
    k = np.array(gj["k"], np.float32)[None, :, None, :]
    q = np.array(gj["q"], np.float32)[None, :, None, :]
    v = np.array(gj["v"], np.float32)[None, :, None, :]
    g = np.array(gj["g"], np.float32)[None, :, None]
    b = np.array(gj["beta"], np.float32)[None, :, None]
    S0 = np.array(gj["S0_rc"], np.float32)
    state = S0.T[None, None]                           # [c][r] layout
    parent = np.array(gj["parent"], np.int32)[None]
    return q, k, v, g, b, state, parent, np.array([3], np.int32)


def test_handworked_tree(golden_dir):
    gj = _handworked(golden_dir)
    q, k, v, g, b, state, parent, n = _single(gj)
    out, delta, states = lin_tree_verify(q, k, v, g, b, state, parent, n, 1.0, "f32", return_states=True)
    # inputs 0.6/0.8 are fp32-rounded, so compare to the exact fractions at fp32 input precision
    np.testing.assert_allclose(out[0, :, 0], gj["expect_out"], atol=1e-6)
    np.testing.assert_allclose(delta[0, :, 0], gj["expect_delta"], atol=1e-6)
    for i in range(3):
        np.testing.assert_allclose(states[0][0][i], gj["expect_state_rc"][i], atol=1e-6)


def test_handworked_commit(golden_dir):
    gj = _handworked(golden_dir)
    q, k, v, g, b, state, parent, n = _single(gj)
    for c in gj["commit"]:
        path = np.array(c["path"], np.int32)[None]
        L = np.array([len(c["path"])], np.int32)
        new = lin_commit_replay(state, path, L, k, v, g, b, parent, n, "f32")
        np.testing.assert_allclose(new[0, 0].T, c["expect_state_rc"], atol=1e-6)


def _random_problem(seed, n=8, Hk=2, Hv=4, dk=8, dv=6, kind="small"):
    rng = np.random.default_rng(seed)
    if kind == "small":
        parent = tree_small(rng)[:n]
    elif kind == "chain":
        parent = tree_chain(n)
    else:
        parent = tree_ddtree(rng, budget=n)
        n = len(parent)
    q = rng.standard_normal((1, n, Hk, dk)).astype(np.float32)
    k = rng.standard_normal((1, n, Hk, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((1, n, Hv, dv)).astype(np.float32)
    g = rng.uniform(0.2, 1.0, (1, n, Hv)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, (1, n, Hv)).astype(np.float32)
    state = rng.normal(0, 0.5, (1, Hv, dv, dk)).astype(np.float32)
    return q, k, v, g, b, state, parent[None].astype(np.int32), np.array([n], np.int32)


def test_identity_gate_keeps_state():
    """g = 1, beta = 0: no update, so o_i = scale * S0^T q_i and commit leaves S0 exactly."""
    q, k, v, g, b, state, parent, n = _random_problem(1)
    g[:] = 1.0
    b[:] = 0.0
    out, delta = lin_tree_verify(q, k, v, g, b, state, parent, n, 0.5)
    Hk, Hv = q.shape[2], v.shape[2]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        S0 = state[0, h].T.astype(np.float64)
        np.testing.assert_allclose(out[0, :, h], 0.5 * q[0, :, kh].astype(np.float64) @ S0, atol=1e-12)
    assert np.all(delta == 0)
    path = np.array([root_path(parent[0], 5)], np.int32)
    new = lin_commit_replay(state, path, np.array([path.shape[1]], np.int32), k, v, g, b, parent, n)
    assert np.array_equal(new, state.astype(np.float64))


def test_zero_gate_forgets_parent():
    """g = 0: S_i = k_i (beta_i v_i)^T, so o_i = scale * beta_i (k_i . q_i) v_i."""
    q, k, v, g, b, state, parent, n = _random_problem(2)
    g[:] = 0.0
    out, delta = lin_tree_verify(q, k, v, g, b, state, parent, n, 0.25)
    Hk, Hv = q.shape[2], v.shape[2]
    for i in range(int(n[0])):
        for h in range(Hv):
            kh = h // (Hv // Hk)
            kq = float(k[0, i, kh].astype(np.float64) @ q[0, i, kh].astype(np.float64))
            want = 0.25 * float(b[0, i, h]) * kq * v[0, i, h].astype(np.float64)
            np.testing.assert_allclose(out[0, i, h], want, atol=1e-12)


def test_one_hot_key_writes_row():
    """k = e_r and beta = 1: row r of S_i becomes v_i; the other rows are g_i times the parent's."""
    q, k, v, g, b, state, parent, n = _random_problem(3, dk=5, dv=7)
    rng = np.random.default_rng(3)
    k[:] = 0
    rows = rng.integers(0, 5, size=k.shape[:3])
    for i in range(k.shape[1]):
        for kh in range(k.shape[2]):
            k[0, i, kh, rows[0, i, kh]] = 1.0
    b[:] = 1.0
    _, _, states = lin_tree_verify(q, k, v, g, b, state, parent, n, 1.0, return_states=True)
    Hk, Hv = q.shape[2], v.shape[2]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        for i in range(int(n[0])):
            p = int(parent[0, i])
            Sp = state[0, h].T.astype(np.float64) if p < 0 else states[0][h][p]
            r = rows[0, i, kh]
            Si = states[0][h][i]
            np.testing.assert_allclose(Si[r], v[0, i, h], atol=1e-12)
            others = [x for x in range(5) if x != r]
            np.testing.assert_allclose(Si[others], g[0, i, h] * Sp[others], atol=1e-12)


def test_delta_rule_identity():
    """For every node: S_i^T k_i = (1 - beta |k|^2) g S_p^T k_i + beta |k|^2 v_i (the state
    moves its prediction for k_i a fraction beta|k|^2 of the way to v_i)."""
    q, k, v, g, b, state, parent, n = _random_problem(4, n=8)
    k *= np.float32(1.3)   # not unit norm, so the |k|^2 factor matters
    _, _, states = lin_tree_verify(q, k, v, g, b, state, parent, n, 1.0, return_states=True)
    Hk, Hv = q.shape[2], v.shape[2]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        for i in range(int(n[0])):
            p = int(parent[0, i])
            Sp = state[0, h].T.astype(np.float64) if p < 0 else states[0][h][p]
            ki = k[0, i, kh].astype(np.float64)
            kk = ki @ ki
            bb, gg = float(b[0, i, h]), float(g[0, i, h])
            want = (1 - bb * kk) * gg * (Sp.T @ ki) + bb * kk * v[0, i, h]
            np.testing.assert_allclose(states[0][h][i].T @ ki, want, atol=1e-12)


def test_chain_matches_transition_matrix_form():
    """A chain is a degenerate tree (PR #606, "Paper mapping").  Along a chain the state is
    S_t = A_t S_{t-1} + beta_t k_t v_t^T with A_t = g_t (I - beta_t k_t k_t^T); this
    product-of-transitions form is computed here with explicit dk x dk matrices."""
    n = 7
    q, k, v, g, b, state, parent, nn = _random_problem(5, n=n, kind="chain")
    out, _, states = lin_tree_verify(q, k, v, g, b, state, parent, nn, 0.7, return_states=True)
    Hk, Hv, dk = q.shape[2], v.shape[2], q.shape[3]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        S = state[0, h].T.astype(np.float64)
        for t in range(n):
            kt = k[0, t, kh].astype(np.float64)
            A = g[0, t, h] * (np.eye(dk) - b[0, t, h] * np.outer(kt, kt))
            S = A @ S + b[0, t, h] * np.outer(kt, v[0, t, h])
            np.testing.assert_allclose(states[0][h][t], S, atol=1e-12)
            np.testing.assert_allclose(out[0, t, h], 0.7 * S.T @ q[0, t, kh], atol=1e-12)


@pytest.mark.parametrize("seed,kind", [(6, "small"), (7, "ddtree"), (8, "ddtree")])
def test_tree_equals_per_path_replay(seed, kind):
    """Brute force: node i's output equals the chain recurrence replayed over root_path(i)."""
    q, k, v, g, b, state, parent, n = _random_problem(seed, n=22 if kind == "ddtree" else 8, kind=kind)
    out, delta = lin_tree_verify(q, k, v, g, b, state, parent, n, 0.3)
    Hk, Hv = q.shape[2], v.shape[2]
    f = lambda a: a.astype(np.float64)
    for i in range(int(n[0])):
        path = root_path(parent[0], i)
        for h in range(Hv):
            kh = h // (Hv // Hk)
            o, _ = lin_chain_recurrence(f(q[0, path, kh]), f(k[0, path, kh]), f(v[0, path, h]),
                                        f(g[0, path, h]), f(b[0, path, h]), f(state[0, h].T), 0.3)
            np.testing.assert_allclose(out[0, i, h], o[-1], atol=1e-12)


def test_relabeling_invariance():
    """Numbering the same tree in another topological order permutes the outputs."""
    q, k, v, g, b, state, parent, n = _random_problem(9, n=22, kind="ddtree")
    n0 = int(n[0])
    # breadth-first renumbering of the same tree
    children = [[] for _ in range(n0)]
    for i in range(1, n0):
        children[parent[0, i]].append(i)
    order, frontier = [0], [0]
    while frontier:
        nxt = []
        for x in frontier:
            nxt.extend(sorted(children[x], reverse=True))
        order.extend(nxt)
        frontier = nxt
    order = np.array(order)
    new_of = np.empty(n0, int)
    new_of[order] = np.arange(n0)
    parent2 = np.array([[-1] + [new_of[parent[0, o]] for o in order[1:]]], np.int32)
    out1, d1 = lin_tree_verify(q, k, v, g, b, state, parent, n, 0.5)
    out2, d2 = lin_tree_verify(q[:, order], k[:, order], v[:, order], g[:, order], b[:, order],
                               state, parent2, n, 0.5)
    np.testing.assert_allclose(out2, out1[:, order], atol=1e-12)
    np.testing.assert_allclose(d2, d1[:, order], atol=1e-12)


def test_commit_equals_verify_state_at_path_end():
    """Committing a root path gives the state verify reached at its last node."""
    q, k, v, g, b, state, parent, n = _random_problem(10, n=22, kind="ddtree")
    _, _, states = lin_tree_verify(q, k, v, g, b, state, parent, n, 1.0, return_states=True)
    rng = np.random.default_rng(10)
    for _ in range(4):
        path = random_root_leaf_path(rng, parent[0], int(n[0]))
        for L in range(1, len(path) + 1):
            new = lin_commit_replay(state, path[None, :L], np.array([L], np.int32), k, v, g, b, parent, n)
            for h in range(v.shape[2]):
                np.testing.assert_allclose(new[0, h].T, states[0][h][path[L - 1]], atol=1e-12)


def test_head_grouping():
    """Contiguous grouping: value head h reads key head h // (Hv/Hk); tiled: h % Hk."""
    q, k, v, g, b, state, parent, n = _random_problem(11, Hk=2, Hv=6)
    for mode, kh_of in (("contiguous", lambda h: h // 3), ("tiled", lambda h: h % 2)):
        out, _ = lin_tree_verify(q, k, v, g, b, state, parent, n, 1.0, head_group=mode)
        for h in range(6):
            kh = kh_of(h)
            o1, _ = lin_tree_verify(q[:, :, kh:kh + 1], k[:, :, kh:kh + 1], v[:, :, h:h + 1],
                                    g[:, :, h:h + 1], b[:, :, h:h + 1], state[:, h:h + 1], parent, n, 1.0)
            np.testing.assert_allclose(out[:, :, h], o1[:, :, 0], atol=1e-12)


def test_bf16_inputs_decode_exactly():
    x = np.array([1.0, -2.5, 3.140625, 1e-3, 65504.0], np.float32)
    bits = f32_to_bf16_bits(x)
    got = bf16_bits_to_f64(bits)
    # bf16 keeps 8 significant bits; these values are exact or within half an ulp
    np.testing.assert_allclose(got, x, rtol=2 ** -8)
    assert got[0] == 1.0 and got[1] == -2.5 and got[2] == 3.140625


def test_generated_workload_runs():
    parents, paths = trees_for(1, 2, "ddtree")
    L = gen_lin(1, parents, paths, 2, 6, 16, 16, "bf16")
    out, delta = lin_tree_verify(L.q, L.k, L.v, L.g, L.beta, L.state, L.parent, L.n_nodes, L.scale, "bf16")
    assert np.isfinite(out).all() and np.isfinite(delta).all()
    new = lin_commit_replay(L.state, L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes, "bf16")
    assert np.isfinite(new).all()


def test_empty_path_commits_nothing():
    q, k, v, g, b, state, parent, n = _random_problem(12)
    path = np.array([[0, 1]], np.int32)
    new = lin_commit_replay(state, path, np.array([0], np.int32), k, v, g, b, parent, n)
    assert np.array_equal(new, state.astype(np.float64))


def test_verify_commit_is_commit_then_verify_and_matches_a_chain_replay():
    """lin_tree_verify_commit: the previous step's path committed, then this step's tree
    verified from the stored (fp32) committed state.  Pinned against (i) an empty previous
    path (plain verify), and (ii) two chain steps, whose accepted prefix followed by the
    new chain is one sequential recurrence over all the tokens."""
    from workloads import gen_lin, tree_chain
    rng = np.random.default_rng(11)
    Hk, Hv, dk, dv = 1, 2, 16, 16
    p1, p2 = tree_chain(6), tree_chain(5)
    L1 = gen_lin(70, [p1], [np.arange(4, dtype=np.int32)], Hk, Hv, dk, dv, "f32")
    L2 = gen_lin(71, [p2], [np.arange(5, dtype=np.int32)], Hk, Hv, dk, dv, "f32")
    prev = (L1.path, L1.path_len, L1.k, L1.v, L1.g, L1.beta, L1.parent, L1.n_nodes)
    st, out, delta = oracle.lin_tree_verify_commit(L1.state, prev, L2.q, L2.k, L2.v, L2.g, L2.beta, L2.parent,
                                                   L2.n_nodes, L2.scale, "f32")
    # (ii) one chain: the 4 accepted tokens of step 1, then the 5 tokens of step 2
    for h in range(Hv):
        q = np.concatenate([L1.q[0, :4, 0], L2.q[0, :, 0]]).astype(np.float64)
        k = np.concatenate([L1.k[0, :4, 0], L2.k[0, :, 0]]).astype(np.float64)
        v = np.concatenate([L1.v[0, :4, h], L2.v[0, :, h]]).astype(np.float64)
        g = np.concatenate([L1.g[0, :4, h], L2.g[0, :, h]]).astype(np.float64)
        bt = np.concatenate([L1.beta[0, :4, h], L2.beta[0, :, h]]).astype(np.float64)
        o_ref, S_end = oracle.lin_chain_recurrence(q, k, v, g, bt, L1.state[0, h].T.astype(np.float64), L2.scale)
        np.testing.assert_allclose(out[0, :, h], o_ref[4:], rtol=1e-6, atol=1e-6)   # fp32 stored state
    # (i) nothing accepted in the previous step: the state is unchanged and the verify is plain
    prev0 = (L1.path, np.zeros(1, np.int32), L1.k, L1.v, L1.g, L1.beta, L1.parent, L1.n_nodes)
    st0, out0, _ = oracle.lin_tree_verify_commit(L1.state, prev0, L2.q, L2.k, L2.v, L2.g, L2.beta, L2.parent,
                                                 L2.n_nodes, L2.scale, "f32")
    ref0, _ = oracle.lin_tree_verify(L2.q, L2.k, L2.v, L2.g, L2.beta, L1.state, L2.parent, L2.n_nodes, L2.scale, "f32")
    assert np.array_equal(st0, L1.state.astype(np.float64))
    np.testing.assert_allclose(out0, ref0, rtol=1e-15, atol=1e-15)


def _chain_step(cfg, n, L, Hk=1, Hv=2, dk=16, dv=16, dtype="f32"):
    from workloads import gen_lin, tree_chain
    return gen_lin(cfg, [tree_chain(n)], [np.arange(L, dtype=np.int32)], Hk, Hv, dk, dv, dtype)


def _prev(L):
    return (L.path, L.path_len, L.k, L.v, L.g, L.beta, L.parent, L.n_nodes)


def test_bank_of_chain_steps_is_one_chain():
    """Three accepted chain steps pending (4, 0 and 6 tokens accepted), then a fourth chain
    verified: one sequential recurrence over the accepted tokens followed by the new chain
    (a chain is a degenerate tree, PR #606 "Paper mapping")."""
    steps = [_chain_step(80, 6, 4), _chain_step(81, 5, 1), _chain_step(82, 7, 6)]
    steps[1].path_len[:] = 0                         # the middle step accepted nothing
    last = _chain_step(83, 5, 5)
    S0 = steps[0].state
    st, out, delta = oracle.lin_tree_verify_bank(S0, [_prev(s) for s in steps], last.q, last.k, last.v, last.g,
                                                 last.beta, last.parent, last.n_nodes, last.scale, "f32")
    acc = [(s, int(s.path_len[0])) for s in steps]
    for h in range(last.Hv):
        cat = lambda f, hh: np.concatenate([f(s)[0, :L, hh] for s, L in acc] + [f(last)[0, :, hh]]).astype(np.float64)
        q, k = cat(lambda s: s.q, 0), cat(lambda s: s.k, 0)
        v, g, bt = cat(lambda s: s.v, h), cat(lambda s: s.g, h), cat(lambda s: s.beta, h)
        o_ref, _ = oracle.lin_chain_recurrence(q, k, v, g, bt, S0[0, h].T.astype(np.float64), last.scale)
        n_acc = sum(L for _, L in acc)
        np.testing.assert_allclose(out[0, :, h], o_ref[n_acc:], rtol=1e-6, atol=1e-6)   # fp32 stored states
        # the committed state is the chain's state after the accepted tokens
        _, S_acc = oracle.lin_chain_recurrence(q[:n_acc], k[:n_acc], v[:n_acc], g[:n_acc], bt[:n_acc],
                                               S0[0, h].T.astype(np.float64), last.scale)
        np.testing.assert_allclose(st[0, h].T, S_acc, rtol=1e-6, atol=1e-6)


def test_bank_factor_form():
    """The pending bank's closed form: with the entries e of every pending step's accepted
    path in acceptance order, each carrying the key k_e, decay g_e and the delta delta_e that
    step's verify captured,  S = (prod_e g_e) S0 + sum_e (prod_{e' > e} g_e') k_e delta_e^T.
    Built here entry by entry with explicit products; the steps are 22-node trees."""
    from workloads import gen_lin, trees_for
    Hk, Hv, dk, dv = 2, 4, 16, 8
    steps = [gen_lin(90 + t, *trees_for(90 + t, 1, "ddtree"), Hk, Hv, dk, dv, "f32") for t in range(3)]
    S0 = steps[0].state
    # every step's captured deltas, from the state the bank oracle commits before it
    entries = []                                     # per value head: (k_e, g_e, delta_e)
    for t, s in enumerate(steps):
        st, _, delta = oracle.lin_tree_verify_bank(S0, [_prev(x) for x in steps[:t]], s.q, s.k, s.v, s.g, s.beta,
                                                   s.parent, s.n_nodes, s.scale, "f32")
        for a in s.path[0, :int(s.path_len[0])]:
            entries.append((s.k[0, a], s.g[0, a], delta[0, a]))
    last = gen_lin(99, *trees_for(99, 1, "ddtree"), Hk, Hv, dk, dv, "f32")
    st, _, _ = oracle.lin_tree_verify_bank(S0, [_prev(x) for x in steps], last.q, last.k, last.v, last.g,
                                           last.beta, last.parent, last.n_nodes, last.scale, "f32")
    assert len(entries) > 6
    for h in range(Hv):
        kh = h // (Hv // Hk)
        G = np.prod([float(g[h]) for _, g, _ in entries])
        S = G * S0[0, h].T.astype(np.float64)
        for e, (ke, _, de) in enumerate(entries):
            c = np.prod([float(g[h]) for _, g, _ in entries[e + 1:]])
            S += c * np.outer(ke[kh].astype(np.float64), de[h])
        np.testing.assert_allclose(st[0, h].T, S, rtol=1e-5, atol=1e-6)


def test_bank_degenerate_cases():
    """Nothing pending: the plain verify.  Only empty paths pending: the state is unchanged
    bit for bit."""
    from workloads import gen_lin, trees_for
    s1 = gen_lin(95, *trees_for(95, 2, "ddtree"), 2, 4, 16, 16, "bf16")
    s2 = gen_lin(96, *trees_for(96, 2, "ddtree"), 2, 4, 16, 16, "bf16")
    st, out, delta = oracle.lin_tree_verify_bank(s1.state, [], s2.q, s2.k, s2.v, s2.g, s2.beta, s2.parent,
                                                 s2.n_nodes, s2.scale, "bf16")
    ref_o, ref_d = oracle.lin_tree_verify(s2.q, s2.k, s2.v, s2.g, s2.beta, s1.state, s2.parent, s2.n_nodes,
                                          s2.scale, "bf16")
    assert np.array_equal(st, s1.state.astype(np.float64))
    np.testing.assert_array_equal(out, ref_o)
    np.testing.assert_array_equal(delta, ref_d)
    p = _prev(s1)
    empty = (p[0], np.zeros_like(p[1])) + p[2:]
    st2, out2, _ = oracle.lin_tree_verify_bank(s1.state, [empty, empty], s2.q, s2.k, s2.v, s2.g, s2.beta, s2.parent,
                                               s2.n_nodes, s2.scale, "bf16")
    assert np.array_equal(st2, s1.state.astype(np.float64))
    np.testing.assert_array_equal(out2, ref_o)

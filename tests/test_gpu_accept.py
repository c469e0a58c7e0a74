"""Parity of the HIP greedy acceptance and KV compaction against the oracle.

Everything here is index or byte work, so the bar is bit-exact: the argmax of every node,
the accepted path, its length and the next token must equal the oracle's; the compacted
caches must equal the oracle's byte for byte.  Both sides decide the argmax on the logits'
own values (bf16 or fp32), exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import tree_verify_linear_amd as tvl
from tvutil import t_bits, t_f32, t_i32, t_u8
from workloads import (gen_accept, workload_accept, trees_for, tree_chain, tree_ddtree, pad_trees, pad_paths,
                       random_root_leaf_path, row_bytes)

pytestmark = pytest.mark.gpu


def run_accept(A, sentinel=True):
    lg = t_bits(A.logits) if A.dtype == "bf16" else t_f32(A.logits)
    B, N = A.parent.shape
    outs = None
    if sentinel:
        outs = dict(target=torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
                    path=torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
                    path_len=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
                    next_token=torch.full((B,), -7, dtype=torch.int32, device="cuda"))
    r = tvl.tree_accept_greedy(lg, t_i32(A.parent), t_i32(A.n_nodes), t_i32(A.tokens), **(outs or {}))
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in r]


def check_accept(A, label=""):
    tgt, path, plen, nxt = run_accept(A)
    rt, rp, rl, rn = oracle.tree_accept_greedy(A.logits, A.dtype, A.parent, A.n_nodes, A.tokens)
    print(f"[accept {label}] B={A.parent.shape[0]} V={A.V} {A.dtype}: path lengths {np.bincount(rl).tolist()}")
    assert np.array_equal(tgt, rt), f"argmax differs at {np.argwhere(tgt != rt)[:5].tolist()}"
    assert np.array_equal(path, rp)
    assert np.array_equal(plen, rl)
    assert np.array_equal(nxt, rn)
    return tgt, path, plen, nxt


def test_accept_batched_full_vocab():
    """64 sequences of 22-node trees, vocabulary 151936, bf16 logits: every row exact."""
    A = workload_accept(64)
    _, _, plen, _ = check_accept(A, "b64")
    assert plen.max() > 2, "the workload should accept more than the root on some sequence"


def test_accept_f32_and_ties():
    """fp32 logits; half the rows carry an exact tie for the maximum (the lower index wins)."""
    parents, _ = trees_for(83, 8, "ddtree")
    check_accept(gen_accept(83, parents, 151936, "f32", tie_p=0.5), "f32 ties")
    check_accept(gen_accept(84, parents, 151936, "bf16", tie_p=0.5), "bf16 ties")


@pytest.mark.parametrize("V", [1, 7, 8, 9, 4099, 16383, 16384, 16385, 50021, 32768 + 13])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accept_vocab_tails(V, dtype):
    """Vocabularies that end mid-vector and mid-chunk, and odd ones whose rows are not
    16-byte aligned (read one logit at a time)."""
    rng = np.random.default_rng(V)
    parents = [tree_ddtree(rng, budget=22), tree_chain(5), np.array([-1], np.int32)]
    check_accept(gen_accept(85, parents, V, dtype, match_p=0.9, tie_p=0.3), f"V{V}")


def _special_rows(dtype):
    """Rows whose argmax rests on NaN, infinities and signed zeros."""
    V = 20000
    rows = []
    nan, inf = np.float32(np.nan), np.float32(np.inf)
    r = np.full(V, nan, np.float32); rows.append(r)                           # all NaN -> 0
    r = np.full(V, -inf, np.float32); r[:5] = nan; rows.append(r)             # -> 5
    r = np.full(V, -1.0, np.float32); r[17000] = 0.0; r[300] = -0.0; rows.append(r)   # -> 300
    r = np.full(V, -1.0, np.float32); r[9000] = inf; r[12000] = inf; r[4] = nan; rows.append(r)  # -> 9000
    r = np.full(V, nan, np.float32); r[19999] = -3.0; rows.append(r)          # -> 19999
    r = np.full(V, 1.0, np.float32); rows.append(r)                           # -> 0
    r = np.random.default_rng(1).standard_normal(V).astype(np.float32); r[16384] = 50; r[16385] = 50; rows.append(r)
    x = np.stack(rows)
    if dtype == "bf16":
        return (x.view(np.uint32) >> 16).astype(np.uint16)
    return x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_accept_nan_inf_signed_zero(dtype):
    x = _special_rows(dtype)
    n = x.shape[0]
    parent = np.array([[-1] + list(range(n - 1))], np.int32)                  # a chain of n nodes
    tokens = np.array([[0, 0, 5, 300, 9000, 19999, 0]], np.int32)        # every step matches
    from workloads import AcceptInputs
    A = AcceptInputs(dtype, x[None], tokens, parent, np.array([n], np.int32), x.shape[1])
    tgt, path, plen, nxt = check_accept(A, f"special {dtype}")
    assert tgt[0].tolist() == [0, 5, 300, 9000, 19999, 0, 16384]
    assert plen[0] == n and nxt[0] == 16384


def test_accept_ragged_chains_and_rejections():
    """A full chain accepted to its end, a root with no matching child, a 64-node tree, and
    padding rows beyond each tree (target and path padded with -1)."""
    rng = np.random.default_rng(5)
    parents = [tree_chain(12), tree_ddtree(rng, budget=64, max_depth=16, topk=6), np.array([-1], np.int32),
               tree_ddtree(rng, budget=9)]
    A = gen_accept(86, parents, 3000, "bf16", match_p=1.0)
    tgt, path, plen, nxt = check_accept(A, "ragged")
    assert plen[0] == 12 and plen[2] == 1
    assert (tgt[2, 1:] == -1).all() and (path[2, 1:] == -1).all()


def test_accept_deterministic_and_batch_invariant():
    A = workload_accept(6, V=40000)
    r1 = run_accept(A)
    r2 = run_accept(A)
    assert all(np.array_equal(a, b) for a, b in zip(r1, r2))
    one = workload_accept(1, V=40000, seq_ids=[3])
    r3 = run_accept(one)
    assert np.array_equal(r3[0][0], r1[0][3]) and np.array_equal(r3[1][0], r1[1][3])


def _gen_caches(seed, B, Hkv, Tcap, D, kt, vt):
    rng = np.random.default_rng(seed)
    k = rng.integers(0, 256, size=(B, Hkv, Tcap, row_bytes(kt, D)), dtype=np.uint8)
    v = rng.integers(0, 256, size=(B, Hkv, Tcap, row_bytes(vt, D)), dtype=np.uint8)
    return k, v


def check_compact(k, v, kt, vt, n_past, path, path_len, label=""):
    dk, dv = t_u8(k), t_u8(v)
    tvl.kv_tree_compact(dk, dv, kt, vt, t_i32(n_past), t_i32(path), t_i32(path_len))
    torch.cuda.synchronize()
    rk = oracle.kv_compact(k, n_past, path, path_len)
    rv = oracle.kv_compact(v, n_past, path, path_len)
    gk, gv = dk.cpu().numpy(), dv.cpu().numpy()
    moved = int(sum(int(np.sum(np.asarray(path[b][:path_len[b]]) != np.arange(path_len[b]))) for b in range(len(n_past))))
    print(f"[compact {label}] {kt}/{vt} rows moved per head: {moved}")
    assert np.array_equal(gk, rk), "K cache differs"
    assert np.array_equal(gv, rv), "V cache differs"


def test_compact_accepted_paths():
    """The batched step's caches (4 KV heads, D=256, Q8_0) after the acceptance of its
    trees: accepted rows move to n_past + m, everything else is untouched."""
    A = workload_accept(64, V=2048)
    _, rp, rl, _ = oracle.tree_accept_greedy(A.logits, A.dtype, A.parent, A.n_nodes, A.tokens)
    B, N = A.parent.shape
    rng = np.random.default_rng(7)
    n_past = rng.integers(0, 300, size=B).astype(np.int32)
    k, v = _gen_caches(1, B, 4, 300 + N, 256, "q8_0", "q8_0")
    check_compact(k, v, "q8_0", "q8_0", n_past, rp.astype(np.int32), rl.astype(np.int32), "accepted")


@pytest.mark.parametrize("kt,vt,D", [("q4_0", "q4_0", 256), ("q8_0", "q4_0", 256), ("q4_0", "q8_0", 128),
                                     ("q8_0", "q8_0", 32), ("q8_0", "q4_0", 512)])
def test_compact_overlapping_moves(kt, vt, D):
    """Random root paths on random trees, so that sources are overwritten by other moves
    (a path 0, 2, 3 reads slot 2 before it receives slot 3); other head sizes take the
    2-byte copy path."""
    rng = np.random.default_rng(D + len(kt))
    parents = [tree_ddtree(rng, budget=22), tree_chain(20), tree_ddtree(rng, budget=64, max_depth=16, topk=6),
               np.array([-1], np.int32)]
    parent, n = pad_trees(parents)
    paths = [random_root_leaf_path(rng, parent[b], int(n[b])) for b in range(len(parents))]
    paths[1] = np.array([0, 2, 3, 5, 9], np.int32)                 # not a tree path: a plain move list
    path, plen = pad_paths(paths, lmax=parent.shape[1])
    n_past = np.array([5, 0, 100, 17], np.int32)
    k, v = _gen_caches(2, len(parents), 3, 180, D, kt, vt)
    check_compact(k, v, kt, vt, n_past, path, plen, f"overlap D{D}")


def test_compact_empty_and_identity():
    """path_len 0 and identity paths (a chain accepted in order) leave the caches unchanged."""
    B = 3
    path = np.tile(np.arange(8, dtype=np.int32), (B, 1))
    plen = np.array([0, 8, 1], np.int32)
    n_past = np.array([0, 10, 50], np.int32)
    k, v = _gen_caches(3, B, 2, 64, 256, "q8_0", "q4_0")
    check_compact(k, v, "q8_0", "q4_0", n_past, path, plen, "identity")

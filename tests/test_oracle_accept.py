"""Pins of the greedy-acceptance and KV-compaction oracle (CPU only).

Hand-worked walks and argmax rows (tests/golden/accept_handworked.json), a hand-built cache
for the compaction (including the overlap where a destination slot is a later source), and
invariants that hold for any input: the walk returns a root path whose every step matches
the target's prediction, and it is maximal (no child of the last node matches).
"""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import f32_to_bf16_bits, gen_accept, trees_for, tree_ddtree


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "accept_handworked.json")) as f:
        return json.load(f)


def test_walk_handworked(golden_dir):
    for case in _golden(golden_dir)["cases"]:
        n = len(case["parent"])
        path, L, nxt = oracle.greedy_walk(case["parent"], n, case["tokens"], case["target"])
        assert path == case["path"], case["name"]
        assert L == len(case["path"]) and nxt == case["next_token"], case["name"]


def test_argmax_handworked(golden_dir):
    for case in _golden(golden_dir)["argmax"]:
        vals = np.array([float(v) for v in case["values"]], dtype=np.float32)
        assert int(oracle.argmax_rows(vals[None], "f32")[0]) == case["index"], case
        # the same values as bf16 bit patterns (all are exact in bf16)
        assert int(oracle.argmax_rows(f32_to_bf16_bits(vals)[None], "bf16")[0]) == case["index"], case


def test_argmax_bf16_resolution():
    # 1.0 and the next bf16 value (1 + 2^-7): distinct, the larger wins
    bits = np.array([[0x3F80, 0x3F81, 0x3F80]], dtype=np.uint16)
    assert int(oracle.argmax_rows(bits, "bf16")[0]) == 1


def test_compaction_handworked():
    # one sequence, one KV head, 6 slots of 4 bytes; T = 2; path 0 -> 2 -> 3 moves slot 4 to
    # slot 3 and slot 5 to slot 4 (slot 4 is read before it is overwritten)
    cache = np.arange(6 * 4, dtype=np.uint8).reshape(1, 1, 6, 4)
    out = oracle.kv_compact(cache, [2], [[0, 2, 3]], [3])
    want = cache.copy()
    want[0, 0, 3] = cache[0, 0, 4]
    want[0, 0, 4] = cache[0, 0, 5]
    assert np.array_equal(out, want)
    assert np.array_equal(out[0, 0, :3], cache[0, 0, :3])      # committed slots and the root untouched


def test_walk_invariants_random():
    rng = np.random.default_rng(5)
    parents = [tree_ddtree(rng, budget=22) for _ in range(8)]
    A = gen_accept(11, parents, 512, "bf16", tie_p=0.3)
    tgt, path, plen, nxt = oracle.tree_accept_greedy(A.logits, "bf16", A.parent, A.n_nodes, A.tokens)
    for b in range(len(parents)):
        n, L = int(A.n_nodes[b]), int(plen[b])
        oracle.validate_path(A.parent[b], n, path[b], L)
        for m in range(1, L):
            assert A.tokens[b, path[b, m]] == tgt[b, path[b, m - 1]]
        last = int(path[b, L - 1])
        kids = [c for c in range(1, n) if A.parent[b, c] == last]
        assert all(A.tokens[b, c] != tgt[b, last] for c in kids)      # maximal
        assert nxt[b] == tgt[b, last]
        assert np.all(tgt[b, n:] == -1) and np.all(path[b, L:] == -1)
    assert plen.max() > 2                                            # the planted matches descend


def test_planted_ties_resolve_low():
    rng = np.random.default_rng(6)
    A = gen_accept(12, [tree_ddtree(rng, budget=22)], 256, "f32", tie_p=1.0)
    x = A.logits[0].astype(np.float64)
    for i in range(int(A.n_nodes[0])):
        top = np.flatnonzero(x[i] == x[i].max())
        assert oracle.argmax_rows(A.logits[0, i][None], "f32")[0] == top[0]

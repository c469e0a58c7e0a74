"""The device-side metadata check (tv_check_metadata) against the host validators.

Valid trees and paths give 0; each planted fault gives exactly its bit; on random
corruptions the device mask is 0 exactly when the host validators accept the sequence.
"""
import numpy as np
import pytest
import torch

import tree_verify_linear_amd as tvl
from tvutil import t_i32
from workloads import trees_for, pad_trees, pad_paths

pytestmark = pytest.mark.gpu
BIT = tvl.META_BITS


def _device_masks(parent, n, path=None, plen=None):
    st = tvl.check_metadata(t_i32(parent), t_i32(n), None if path is None else t_i32(path),
                            None if plen is None else t_i32(plen))
    torch.cuda.synchronize()
    return st.cpu().numpy()


def _host_ok(parent, n, path=None, plen=None):
    """Per sequence: do the host validators accept it?"""
    ok = []
    for b in range(parent.shape[0]):
        try:
            if path is None:
                tvl.validate_tree(parent[b:b + 1], n[b:b + 1])
            else:
                tvl.validate_path(parent[b:b + 1], n[b:b + 1], path[b:b + 1], plen[b:b + 1])
            ok.append(True)
        except tvl.TreeVerifyError:
            ok.append(False)
    return np.array(ok)


def test_valid_batches_pass():
    parents, paths = trees_for(3, 64, "ddtree")
    parent, n = pad_trees(parents)
    path, plen = pad_paths(paths)
    assert (_device_masks(parent, n) == 0).all()
    assert (_device_masks(parent, n, path, plen) == 0).all()
    # wide trees and full-length chains
    parents, paths = trees_for(9, 8, "ddtree", budget=64, max_depth=63)
    parent, n = pad_trees(parents, 64)
    path, plen = pad_paths(paths, 64)
    assert (_device_masks(parent, n, path, plen) == 0).all()


def test_each_fault_sets_its_bit():
    parents, paths = trees_for(4, 1, "ddtree")
    parent, n = pad_trees(parents)
    path, plen = pad_paths(paths)
    N, L = parent.shape[1], int(plen[0])
    assert L >= 3
    off = [i for i in range(1, int(n[0])) if i not in set(path[0, :L].tolist())]   # nodes off the path
    assert len(off) >= 2
    cases = []
    # (every bit is judged on its own, with n_nodes clamped to [0, N]: a path on an empty tree is too long)
    p = parent.copy(); nn = n.copy(); nn[0] = 0; cases.append((p, nn, path, plen, BIT["n_nodes"] | BIT["path_len"]))
    p = parent.copy(); nn = n.copy(); nn[0] = N + 1; cases.append((p, nn, path, plen, BIT["n_nodes"]))
    p = parent.copy(); p[0, 0] = 0; cases.append((p, n, path, plen, BIT["root"]))
    p = parent.copy(); p[0, off[0]] = off[0]; cases.append((p, n, path, plen, BIT["parent"]))
    p = parent.copy(); p[0, off[1]] = -3; cases.append((p, n, path, plen, BIT["parent"]))
    pl = plen.copy(); pl[0] = int(n[0]) + 1; cases.append((parent, n, path, pl, BIT["path_len"]))
    pl = plen.copy(); pl[0] = -1; cases.append((parent, n, path, pl, BIT["path_len"]))
    a = path.copy(); a[0, 0] = 1; cases.append((parent, n, a, plen, BIT["path_root"] | BIT["path_step"]))
    a = path.copy(); a[0, 2] = a[0, 1]; cases.append((parent, n, a, plen, BIT["path_step"]))
    a = path.copy(); a[0, L - 1] = 999; cases.append((parent, n, a, plen, BIT["path_step"]))
    for p, nn, a, pl, want in cases:
        got = int(_device_masks(p, nn, a, pl)[0])
        assert got == want, (got, want)
        assert not _host_ok(p, nn, a, pl)[0]


def test_agrees_with_host_validators_on_random_corruptions():
    rng = np.random.default_rng(17)
    parents, paths = trees_for(5, 64, "ddtree")
    parent, n = pad_trees(parents)
    path, plen = pad_paths(paths)
    for trial in range(6):
        p, nn, a, pl = parent.copy(), n.copy(), path.copy(), plen.copy()
        for b in rng.choice(64, 24, replace=False):
            kind = rng.integers(0, 4)
            if kind == 0:
                p[b, rng.integers(0, p.shape[1])] = rng.integers(-2, p.shape[1] + 2)
            elif kind == 1:
                nn[b] = rng.integers(-1, p.shape[1] + 2)
            elif kind == 2:
                a[b, rng.integers(0, a.shape[1])] = rng.integers(-1, p.shape[1] + 1)
            else:
                pl[b] = rng.integers(-1, a.shape[1] + 2)
        dev = _device_masks(p, nn, a, pl)
        host = _host_ok(p, nn, a, pl)
        assert np.array_equal(dev == 0, host), (trial, np.where((dev == 0) != host))
        dev_t = _device_masks(p, nn)
        host_t = _host_ok(p, nn)
        assert np.array_equal(dev_t == 0, host_t)

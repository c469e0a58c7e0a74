"""The C ABI without a GPU: the library loads, exports every declared symbol, and every
argument error is reported on the host before anything is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import tree_verify_linear_amd as tvl
from workloads import trees_for, pad_trees, pad_paths

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "tree_verify.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _header_functions()
    assert {"lin_tree_verify", "lin_tree_commit", "attn_tree_verify", "attn_tree_workspace_bytes",
            "tv_validate_tree", "tv_validate_path", "tv_last_error", "tv_abi_version"} <= set(names)
    L = tvl.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(tvl.EXPORTS), "binding and header disagree"
    assert tvl.abi_version() == 1


def _fake():
    return ctypes.c_void_p(4096)  # never dereferenced: every call below fails its host checks


def _verify_call(**kw):
    a = dict(B=1, N=8, Hk=1, Hv=1, dk=16, dv=16, dtype=0, head_group=0, scale=0.25)
    a.update(kw)
    f = _fake()
    return tvl.lib().lin_tree_verify(a["B"], a["N"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["dtype"],
                                     a["head_group"], a["scale"], *([kw.get("ptr", f)] * 11))


def test_verify_argument_errors():
    L = tvl.lib()
    assert _verify_call(B=0) == tvl.TV_EINVAL
    assert b"positive" in L.tv_last_error()
    assert _verify_call(N=65) == tvl.TV_ERANGE
    assert _verify_call(dk=48) == tvl.TV_EUNSUPPORTED
    assert b"16, 32, 64, 128" in L.tv_last_error()
    assert _verify_call(dv=256) == tvl.TV_EUNSUPPORTED
    assert _verify_call(dtype=7) == tvl.TV_EUNSUPPORTED
    assert _verify_call(Hk=2, Hv=3) == tvl.TV_EINVAL
    assert _verify_call(head_group=5) == tvl.TV_EINVAL
    assert _verify_call(scale=float("nan")) == tvl.TV_EINVAL
    assert _verify_call(ptr=None) == tvl.TV_EINVAL
    assert b"null" in L.tv_last_error()
    assert _verify_call(ptr=ctypes.c_void_p(18)) == tvl.TV_EINVAL      # misaligned
    assert b"aligned" in L.tv_last_error()


def test_commit_argument_errors():
    L = tvl.lib()
    f = _fake()
    assert L.lin_tree_commit(1, 8, 1, 1, 16, 16, 0, 0, f, f, 0, f, f, f, f, f) == tvl.TV_ERANGE   # Lmax 0
    assert L.lin_tree_commit(1, 8, 1, 1, 16, 16, 0, 0, f, f, 9, f, f, f, f, f) == tvl.TV_ERANGE   # Lmax > N
    assert L.lin_tree_commit(1, 8, 1, 1, 16, 16, 0, 0, None, f, 4, f, f, f, f, f) == tvl.TV_EINVAL
    assert L.lin_tree_commit(1, 8, 1, 1, 12, 16, 0, 0, f, f, 4, f, f, f, f, f) == tvl.TV_EUNSUPPORTED
    m = ctypes.c_void_p(4098)                                  # 2-byte aligned only
    for i in range(3):                                         # k, cap_delta, state
        args = [f, f, 4, f, f, f, f, None]
        args[[3, 5, 6][i]] = m
        assert L.lin_tree_commit(1, 8, 1, 1, 16, 16, 1, 0, *args) == tvl.TV_EINVAL
        assert b"aligned" in L.tv_last_error()


def test_bank_argument_errors():
    L = tvl.lib()
    f = _fake()

    def vb(Emax=32, flush=0, ptr=f, bank_k=None, prev_Lmax=4, **kw):
        a = dict(B=1, N=8, Hk=1, Hv=1, dk=16, dv=16, dtype=1, head_group=0)
        a.update(kw)
        return L.lin_tree_verify_bank(a["B"], a["N"], a["Hk"], a["Hv"], a["dk"], a["dv"], a["dtype"],
                                      a["head_group"], 0.25, *([ptr] * 9), ctypes.c_void_p(8192), 8, ptr, ptr,
                                      prev_Lmax, ptr, ptr, ptr, Emax, flush,
                                      bank_k if bank_k is not None else ptr, ptr, ptr, ptr, None)

    assert vb(Emax=48) == tvl.TV_ERANGE and b"multiple of 32" in L.tv_last_error()
    assert vb(Emax=288) == tvl.TV_ERANGE
    assert vb(Emax=0) == tvl.TV_ERANGE
    assert vb(flush=2) == tvl.TV_EINVAL
    assert vb(prev_Lmax=9) == tvl.TV_ERANGE                        # prev_Lmax > prev_N
    assert vb(ptr=None) == tvl.TV_EINVAL and b"null" in L.tv_last_error()
    assert vb(bank_k=ctypes.c_void_p(4104)) == tvl.TV_EINVAL and b"aligned" in L.tv_last_error()
    assert vb(dk=48) == tvl.TV_EUNSUPPORTED

    def fl(Emax=32, ptr=f, bank_delta=None, prev_Lmax=4, state=f):
        return L.lin_bank_flush(1, 1, 1, 16, 16, 1, 0, state, 8, ptr, ptr, prev_Lmax, ptr, ptr, ptr, Emax, ptr, ptr,
                                bank_delta if bank_delta is not None else ptr, ptr, None)

    assert fl(Emax=40) == tvl.TV_ERANGE
    assert fl(prev_Lmax=0) == tvl.TV_ERANGE
    assert fl(ptr=None) == tvl.TV_EINVAL
    assert fl(state=ctypes.c_void_p(4100)) == tvl.TV_EINVAL and b"aligned" in L.tv_last_error()
    assert fl(bank_delta=ctypes.c_void_p(4100)) == tvl.TV_EINVAL and b"aligned" in L.tv_last_error()


def test_metadata_check_argument_errors():
    L = tvl.lib()
    f = _fake()
    assert L.tv_check_metadata(None, f, None, None, 1, 8, 1, f, None) == tvl.TV_EINVAL
    assert L.tv_check_metadata(f, f, f, None, 1, 8, 1, f, None) == tvl.TV_EINVAL      # path without path_len
    assert b"both" in L.tv_last_error()
    assert L.tv_check_metadata(f, f, None, None, 0, 8, 1, f, None) == tvl.TV_EINVAL
    assert L.tv_check_metadata(f, f, None, None, 1, 65, 1, f, None) == tvl.TV_ERANGE
    assert L.tv_check_metadata(f, f, f, f, 1, 8, 9, f, None) == tvl.TV_ERANGE        # Lmax > N
    assert L.tv_check_metadata(f, f, f, f, 1, 8, 0, f, None) == tvl.TV_ERANGE


def test_attention_argument_errors():
    L = tvl.lib()
    f = _fake()
    base = [1, 22, 24, 4, 256, 4200, 0, 0, 2048, 0.0625]

    def call(**kw):
        a = list(base)
        for i, key in enumerate(["B", "N", "Hq", "Hkv", "D", "Tcap", "kt", "vt", "W", "scale"]):
            if key in kw:
                a[i] = kw[key]
        ws = kw.get("ws", 1 << 30)
        return L.attn_tree_verify(*a, *([kw.get("ptr", f)] * 8), f, ws, None)

    assert call(Hq=25) == tvl.TV_EINVAL
    assert call(Hq=40, Hkv=4) == tvl.TV_EUNSUPPORTED              # 10 query heads per KV head
    assert call(D=192) == tvl.TV_EUNSUPPORTED
    assert call(D=128) == tvl.TV_EUNSUPPORTED
    assert call(kt=2) == tvl.TV_EUNSUPPORTED
    assert b"supported pairs" in L.tv_last_error()
    assert call(W=-1) == tvl.TV_EINVAL
    assert call(N=65) == tvl.TV_ERANGE
    assert call(scale=float("inf")) == tvl.TV_EINVAL
    assert call(ptr=None) == tvl.TV_EINVAL
    need = tvl.attn_tree_workspace_bytes(1, 22, 24, 4, 256, 4200, 2048)
    assert need > 0
    assert call(ws=need - 1) == tvl.TV_ERANGE
    assert b"workspace" in L.tv_last_error()
    assert tvl.attn_tree_workspace_bytes(1, 22, 24, 5, 256, 4200, 2048) == 0


def test_noalloc_attention_argument_errors():
    """The no-allocation variant runs the same host checks and rejects sizes whose split
    partials exceed its built-in scratch, before touching the device."""
    L = tvl.lib()
    f = _fake()

    def call(B=1, N=22, Hq=24, Hkv=4, D=256, Tcap=4200, kt=0, vt=0, W=2048, ptr=f):
        return L.attn_tree_verify_noalloc(B, N, Hq, Hkv, D, Tcap, kt, vt, W, 0.0625, *([ptr] * 8), None)

    assert call(Hq=25) == tvl.TV_EINVAL
    assert call(D=128) == tvl.TV_EUNSUPPORTED
    assert call(kt=3) == tvl.TV_EUNSUPPORTED and b"supported pairs" in L.tv_last_error()
    assert call(W=-1) == tvl.TV_EINVAL
    assert call(ptr=None) == tvl.TV_EINVAL
    # a shape whose split partials exceed the 64 MiB scratch (the split plan decides which)
    big = None
    for B in range(1, 160):
        for Hkv in (1, 2, 3, 4):
            for N, G in ((22, 6), (64, 8)):
                if big is None and tvl.attn_tree_workspace_bytes(B, N, G * Hkv, Hkv, 256, 131136, 0) > 64 << 20:
                    big = (B, N, G * Hkv, Hkv)
    assert big is not None
    assert call(B=big[0], N=big[1], Hq=big[2], Hkv=big[3], Tcap=131136, W=0) == tvl.TV_ERANGE
    assert b"scratch" in L.tv_last_error()


def test_validate_tree_and_path():
    parents, paths = trees_for(1, 3, "ddtree")
    parent, n = pad_trees(parents)
    path, L = pad_paths(paths)
    tvl.validate_tree(parent, n)
    tvl.validate_path(parent, n, path, L)

    bad = parent.copy(); bad[1, 5] = 7                       # a later node
    with pytest.raises(tvl.TreeVerifyError) as e:
        tvl.validate_tree(bad, n)
    assert e.value.code == tvl.TV_ETOPO and "parent[1][5]=7" in str(e.value)
    bad = parent.copy(); bad[0, 0] = 0
    with pytest.raises(tvl.TreeVerifyError):
        tvl.validate_tree(bad, n)
    with pytest.raises(tvl.TreeVerifyError):
        tvl.validate_tree(parent, np.array([22, 0, 22], np.int32))
    with pytest.raises(tvl.TreeVerifyError):
        tvl.validate_tree(parent, np.array([22, 23, 22], np.int32))

    badp = path.copy(); badp[0, 0] = 1
    with pytest.raises(tvl.TreeVerifyError) as e:
        tvl.validate_path(parent, n, badp, L)
    assert e.value.code == tvl.TV_EPATH
    # a node that is not the child of its predecessor
    badp = path.copy()
    sib = [i for i in range(1, 22) if parent[2, i] != path[2, 0] and i != path[2, 1]][0]
    badp[2, 1] = sib
    with pytest.raises(tvl.TreeVerifyError):
        tvl.validate_path(parent, n, badp, L)
    with pytest.raises(tvl.TreeVerifyError):
        tvl.validate_path(parent, n, path, L + 30)
    ok0 = np.zeros_like(L)
    tvl.validate_path(parent, n, path, ok0)                # empty paths are allowed


def test_accept_argument_errors():
    L = tvl.lib()
    f = _fake()
    V = 151936

    def call(B=2, N=22, V=V, dtype=1, ptr=f, logits=None, ws=1 << 30):
        lg = f if logits is None else logits
        return L.tree_accept_greedy(B, N, V, dtype, lg, *([ptr] * 7), f, ws, None)

    assert call(B=0) == tvl.TV_EINVAL
    assert call(V=0) == tvl.TV_EINVAL
    assert call(N=65) == tvl.TV_ERANGE
    assert call(dtype=3) == tvl.TV_EUNSUPPORTED
    assert b"TV_BF16" in L.tv_last_error()
    assert call(ptr=None) == tvl.TV_EINVAL
    assert call(logits=ctypes.c_void_p(4098)) == tvl.TV_EINVAL      # misaligned logits
    assert b"aligned" in L.tv_last_error()
    need = tvl.tree_accept_workspace_bytes(2, 22, V)
    # one 64-bit partial per (sequence, node, chunk of 16384 bf16 logits), rounded to 256 bytes
    assert need == -(-2 * 22 * 10 * 8 // 256) * 256
    assert tvl.tree_accept_workspace_bytes(2, 22, V, __import__("torch").float32) == -(-2 * 22 * 19 * 8 // 256) * 256
    assert call(ws=need - 1) == tvl.TV_ERANGE
    assert b"workspace" in L.tv_last_error()
    assert L.tree_accept_workspace_bytes(2, 65, V, 1) == 0
    assert L.tree_accept_workspace_bytes(2, 22, V, 5) == 0


def test_compact_argument_errors():
    L = tvl.lib()
    f = _fake()

    def call(B=2, Hkv=4, D=256, Tcap=4200, kt=0, vt=0, Lmax=22, ptr=f, cache=None):
        c = f if cache is None else cache
        return L.kv_tree_compact(B, Hkv, D, Tcap, kt, vt, ptr, ptr, ptr, Lmax, c, c, None)

    assert call(Hkv=0) == tvl.TV_EINVAL
    assert call(D=48) == tvl.TV_EUNSUPPORTED
    assert call(D=544) == tvl.TV_EUNSUPPORTED
    assert call(vt=4) == tvl.TV_EUNSUPPORTED
    assert b"supported pairs" in L.tv_last_error()
    assert call(Lmax=0) == tvl.TV_ERANGE
    assert call(Lmax=65) == tvl.TV_ERANGE
    assert call(ptr=None) == tvl.TV_EINVAL
    assert call(cache=ctypes.c_void_p(4104)) == tvl.TV_EINVAL
    assert b"aligned" in L.tv_last_error()


def test_conv_argument_errors():
    L = tvl.lib()
    f = _fake()

    def verify(B=2, N=22, C=10240, K=4, dtype=1, act=0, ptr=f, x=None):
        xx = f if x is None else x
        return L.conv_tree_verify(B, N, C, K, dtype, act, ptr, ptr, xx, ptr, ptr, ptr, None)

    assert verify(C=0) == tvl.TV_EINVAL
    assert verify(N=65) == tvl.TV_ERANGE
    assert verify(K=1) == tvl.TV_EUNSUPPORTED and b"2..8" in L.tv_last_error()
    assert verify(K=9) == tvl.TV_EUNSUPPORTED
    assert verify(C=10244) == tvl.TV_EUNSUPPORTED and b"multiple of 8" in L.tv_last_error()
    assert verify(dtype=4) == tvl.TV_EUNSUPPORTED
    assert verify(act=2) == tvl.TV_EINVAL
    assert verify(ptr=None) == tvl.TV_EINVAL
    assert verify(x=ctypes.c_void_p(4100)) == tvl.TV_EINVAL and b"aligned" in L.tv_last_error()
    assert L.conv_tree_commit(2, 22, 10240, 4, 1, f, f, 0, f, f, None) == tvl.TV_ERANGE      # Lmax 0
    assert L.conv_tree_commit(2, 22, 10240, 4, 1, f, f, 23, f, f, None) == tvl.TV_ERANGE     # Lmax > N
    assert L.conv_tree_commit(2, 22, 10240, 4, 1, None, f, 22, f, f, None) == tvl.TV_EINVAL
    assert L.conv_tree_commit(2, 22, 10240, 9, 1, f, f, 22, f, f, None) == tvl.TV_EUNSUPPORTED

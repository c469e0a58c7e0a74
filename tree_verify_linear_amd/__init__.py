"""Python binding of libtreeverify.so -- argument marshalling only.

Every step of the tree-verify path runs in the library's HIP kernels; this module only
checks tensor shapes/dtypes, allocates outputs with PyTorch when the caller does not
pass them, and forwards raw device pointers and the current HIP stream.  If the library
is not built, every call raises: there is no fallback.

Layouts (row-major, innermost last) are those of ``include/tree_verify.h``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["TreeVerifyError", "lib", "lib_path", "lin_tree_verify", "lin_tree_commit", "lin_tree_verify_commit",
           "LinBank", "lin_bank_empty", "lin_tree_verify_bank", "lin_bank_flush", "attn_tree_verify", "attn_tree_verify_noalloc", "attn_tree_workspace_bytes", "tree_accept_greedy",
           "tree_accept_workspace_bytes", "kv_tree_compact", "conv_tree_verify", "conv_tree_commit",
           "validate_tree", "validate_path", "check_metadata",
           "abi_version", "KV_TYPES", "EXPORTS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

TV_OK, TV_EINVAL, TV_EUNSUPPORTED, TV_ERANGE, TV_ETOPO, TV_EPATH, TV_EDEVICE = range(7)
TV_F32, TV_BF16 = 0, 1
HEAD_GROUPS = {"contiguous": 0, "tiled": 1}
KV_TYPES = {"q8_0": 0, "q4_0": 1}
ACTIVATIONS = {"none": 0, "silu": 1}
KV_BLOCK_BYTES = {"q8_0": 34, "q4_0": 18}

_i, _f, _p, _sz = ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
EXPORTS = {
    "lin_tree_verify": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "lin_tree_commit": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p, _p, _p]),
    "lin_tree_verify_commit": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                    _i, _p, _p, _i, _p, _p, _p, _p]),
    "lin_tree_verify_bank": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  _i, _p, _p, _i, _p, _p, _p, _i, _i, _p, _p, _p, _p, _p]),
    "lin_bank_flush": (_i, [_i, _i, _i, _i, _i, _i, _i, _p, _i, _p, _p, _i, _p, _p, _p, _i, _p, _p, _p, _p, _p]),
    "attn_tree_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "attn_tree_verify": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "attn_tree_verify_noalloc": (_i, [_i, _i, _i, _i, _i, _i, _i, _i, _i, _f, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "tree_accept_workspace_bytes": (_sz, [_i, _i, _i, _i]),
    "tree_accept_greedy": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "kv_tree_compact": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p]),
    "conv_tree_verify": (_i, [_i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]),
    "conv_tree_commit": (_i, [_i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p]),
    "tv_check_metadata": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p]),
    "tv_validate_tree": (_i, [_p, _p, _i, _i]),
    "tv_validate_path": (_i, [_p, _p, _p, _p, _i, _i, _i]),
    "tv_last_error": (ctypes.c_char_p, []),
    "tv_abi_version": (_i, []),
}


class TreeVerifyError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[tv status {code}] {message}")
        self.code = code


def lib_path() -> str:
    return os.path.join(_HERE, "libtreeverify.so")


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m tree_verify_linear_amd.build`")
        L = ctypes.CDLL(path)
        for name, (res, args) in EXPORTS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(code: int) -> None:
    if code != TV_OK:
        raise TreeVerifyError(code, lib().tv_last_error().decode())


def abi_version() -> int:
    return lib().tv_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _in_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return TV_BF16
    if t.dtype == torch.float32:
        return TV_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def lin_tree_verify(q, k, v, g, beta, state, parent, n_nodes, scale: float, head_group: str = "contiguous",
                    out=None, cap_delta=None):
    """Gated delta-rule layer over the draft tree.  Returns ``(out, cap_delta)``, fp32
    ``[B][N][Hv][dv]``.  ``state`` (fp32 ``[B][Hv][dv][dk]``) is read, never written."""
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = q.dtype
    _dev(q, "q", dt); _dev(k, "k", dt, (B, N, Hk, dk)); _dev(v, "v", dt, (B, N, Hv, dv))
    _dev(g, "g", dt, (B, N, Hv)); _dev(beta, "beta", dt, (B, N, Hv))
    _dev(state, "state", torch.float32, (B, Hv, dv, dk))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    if cap_delta is None:
        cap_delta = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, (B, N, Hv, dv)); _dev(cap_delta, "cap_delta", torch.float32, (B, N, Hv, dv))
    _check(lib().lin_tree_verify(B, N, Hk, Hv, dk, dv, _in_dtype(q), HEAD_GROUPS[head_group], float(scale),
                                 _ptr(parent), _ptr(n_nodes), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(state), _ptr(out), _ptr(cap_delta), _stream(q.device)))
    return out, cap_delta


def lin_tree_commit(state, path, path_len, k, g, cap_delta, head_group: str = "contiguous"):
    """Move ``state`` in place to the end of each sequence's accepted root path."""
    B, Hv, dv, dk = state.shape
    N, Hk = k.shape[1], k.shape[2]
    Lmax = path.shape[1]
    _dev(state, "state", torch.float32)
    _dev(k, "k", (torch.bfloat16, torch.float32), (B, N, Hk, dk)); _dev(g, "g", k.dtype, (B, N, Hv))
    _dev(cap_delta, "cap_delta", torch.float32, (B, N, Hv, dv))
    _dev(path, "path", torch.int32, (B, Lmax)); _dev(path_len, "path_len", torch.int32, (B,))
    _check(lib().lin_tree_commit(B, N, Hk, Hv, dk, dv, _in_dtype(k), HEAD_GROUPS[head_group], _ptr(path),
                                 _ptr(path_len), Lmax, _ptr(k), _ptr(g), _ptr(cap_delta), _ptr(state),
                                 _stream(state.device)))
    return state


def lin_tree_verify_commit(q, k, v, g, beta, state, parent, n_nodes, scale: float, prev_path, prev_path_len,
                           prev_k, prev_g, prev_cap_delta, head_group: str = "contiguous", out=None, cap_delta=None):
    """The previous step's commit (its path, k, g and captured deltas) applied to ``state`` in
    place, then this step's verify from the committed state.  Returns ``(out, cap_delta)``."""
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = q.dtype
    _dev(q, "q", dt); _dev(k, "k", dt, (B, N, Hk, dk)); _dev(v, "v", dt, (B, N, Hv, dv))
    _dev(g, "g", dt, (B, N, Hv)); _dev(beta, "beta", dt, (B, N, Hv))
    _dev(state, "state", torch.float32, (B, Hv, dv, dk))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    PN = prev_k.shape[1]
    _dev(prev_k, "prev_k", dt, (B, PN, Hk, dk)); _dev(prev_g, "prev_g", dt, (B, PN, Hv))
    _dev(prev_cap_delta, "prev_cap_delta", torch.float32, (B, PN, Hv, dv))
    _dev(prev_path, "prev_path", torch.int32); _dev(prev_path_len, "prev_path_len", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    if cap_delta is None:
        cap_delta = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, (B, N, Hv, dv)); _dev(cap_delta, "cap_delta", torch.float32, (B, N, Hv, dv))
    _check(lib().lin_tree_verify_commit(B, N, Hk, Hv, dk, dv, _in_dtype(q), HEAD_GROUPS[head_group], float(scale),
                                        _ptr(parent), _ptr(n_nodes), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                        _ptr(state), _ptr(out), _ptr(cap_delta), PN, _ptr(prev_path),
                                        _ptr(prev_path_len), prev_path.shape[1], _ptr(prev_k), _ptr(prev_g),
                                        _ptr(prev_cap_delta), _stream(q.device)))
    return out, cap_delta


class LinBank:
    """A pending bank: ``k`` [B][Hk][dk][Emax] (input dtype), ``g`` fp32 [B][Hv][Emax],
    ``delta`` fp32 [B][Hv][dv][Emax] and ``length`` int32 [B] (entries pending per sequence,
    besides the previous step's path)."""

    def __init__(self, k, g, delta, length):
        self.k, self.g, self.delta, self.length = k, g, delta, length
        self.Emax = k.shape[3]


def lin_bank_empty(B: int, Hk: int, Hv: int, dk: int, dv: int, Emax: int, dtype, device) -> LinBank:
    """An empty bank of capacity ``Emax`` (a multiple of 32, at most 256)."""
    return LinBank(torch.zeros((B, Hk, dk, Emax), dtype=dtype, device=device),
                   torch.zeros((B, Hv, Emax), dtype=torch.float32, device=device),
                   torch.zeros((B, Hv, dv, Emax), dtype=torch.float32, device=device),
                   torch.zeros((B,), dtype=torch.int32, device=device))


def _dev_bank(bank: LinBank, B, Hk, Hv, dk, dv, dt):
    E = bank.Emax
    _dev(bank.k, "bank.k", dt, (B, Hk, dk, E)); _dev(bank.g, "bank.g", torch.float32, (B, Hv, E))
    _dev(bank.delta, "bank.delta", torch.float32, (B, Hv, dv, E)); _dev(bank.length, "bank.length", torch.int32, (B,))


def _dev_prev(prev_path, prev_path_len, prev_k, prev_g, prev_cap_delta, B, Hk, Hv, dk, dv, dt):
    PN = prev_k.shape[1]
    _dev(prev_k, "prev_k", dt, (B, PN, Hk, dk)); _dev(prev_g, "prev_g", dt, (B, PN, Hv))
    _dev(prev_cap_delta, "prev_cap_delta", torch.float32, (B, PN, Hv, dv))
    _dev(prev_path, "prev_path", torch.int32); _dev(prev_path_len, "prev_path_len", torch.int32, (B,))
    if prev_path.dim() != 2 or prev_path.shape[0] != B:
        raise ValueError(f"prev_path has shape {tuple(prev_path.shape)}, expected ({B}, Lmax)")
    return PN


def lin_tree_verify_bank(q, k, v, g, beta, state, parent, n_nodes, scale: float, prev_path, prev_path_len,
                         prev_k, prev_g, prev_cap_delta, bank: LinBank, flush: bool = False,
                         head_group: str = "contiguous", out=None, cap_delta=None):
    """Verify from the committed state (``state`` + ``bank`` + the previous step's accepted
    path), then append that path to the bank -- or, when it does not fit or ``flush`` is set,
    store the committed state and empty the bank.  Returns ``(out, cap_delta)``."""
    B, N, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    dt = q.dtype
    _dev(q, "q", dt); _dev(k, "k", dt, (B, N, Hk, dk)); _dev(v, "v", dt, (B, N, Hv, dv))
    _dev(g, "g", dt, (B, N, Hv)); _dev(beta, "beta", dt, (B, N, Hv))
    _dev(state, "state", torch.float32, (B, Hv, dv, dk))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    PN = _dev_prev(prev_path, prev_path_len, prev_k, prev_g, prev_cap_delta, B, Hk, Hv, dk, dv, dt)
    _dev_bank(bank, B, Hk, Hv, dk, dv, dt)
    if out is None:
        out = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    if cap_delta is None:
        cap_delta = torch.empty((B, N, Hv, dv), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, (B, N, Hv, dv)); _dev(cap_delta, "cap_delta", torch.float32, (B, N, Hv, dv))
    _check(lib().lin_tree_verify_bank(B, N, Hk, Hv, dk, dv, _in_dtype(q), HEAD_GROUPS[head_group], float(scale),
                                      _ptr(parent), _ptr(n_nodes), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                      _ptr(state), _ptr(out), _ptr(cap_delta), PN, _ptr(prev_path),
                                      _ptr(prev_path_len), prev_path.shape[1], _ptr(prev_k), _ptr(prev_g),
                                      _ptr(prev_cap_delta), bank.Emax, int(bool(flush)), _ptr(bank.k), _ptr(bank.g),
                                      _ptr(bank.delta), _ptr(bank.length), _stream(q.device)))
    return out, cap_delta


def lin_bank_flush(state, prev_path, prev_path_len, prev_k, prev_g, prev_cap_delta, bank: LinBank,
                   head_group: str = "contiguous"):
    """Store the committed state (``state`` + ``bank`` + the previous step's accepted path)
    into ``state`` and empty the bank."""
    B, Hv, dv, dk = state.shape
    Hk = prev_k.shape[2]
    dt = prev_k.dtype
    _dev(state, "state", torch.float32)
    _dev(prev_k, "prev_k", (torch.bfloat16, torch.float32))
    PN = _dev_prev(prev_path, prev_path_len, prev_k, prev_g, prev_cap_delta, B, Hk, Hv, dk, dv, dt)
    _dev_bank(bank, B, Hk, Hv, dk, dv, dt)
    _check(lib().lin_bank_flush(B, Hk, Hv, dk, dv, _in_dtype(prev_k), HEAD_GROUPS[head_group], _ptr(state), PN,
                                _ptr(prev_path), _ptr(prev_path_len), prev_path.shape[1], _ptr(prev_k),
                                _ptr(prev_g), _ptr(prev_cap_delta), bank.Emax, _ptr(bank.k), _ptr(bank.g),
                                _ptr(bank.delta), _ptr(bank.length), _stream(state.device)))
    return state


def attn_tree_workspace_bytes(B: int, N: int, Hq: int, Hkv: int, D: int, Tcap: int, window: int) -> int:
    return int(lib().attn_tree_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window))


def attn_tree_verify(q, k_cache, v_cache, k_type: str, v_type: str, n_past, parent, n_nodes, window: int,
                     scale: float, out=None, lse=None, workspace=None, want_lse: bool = True):
    """Tree-masked attention over the quantised cache.  Returns ``(out, lse)``: fp32
    ``[B][N][Hq][D]`` and ``[B][N][Hq]`` (``lse`` is None when ``want_lse`` is False)."""
    B, N, Hq, D = q.shape
    Hkv, Tcap = k_cache.shape[1], k_cache.shape[2]
    _dev(q, "q", torch.bfloat16)
    _dev(k_cache, "k_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[k_type]))
    _dev(v_cache, "v_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[v_type]))
    _dev(n_past, "n_past", torch.int32, (B,))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    if out is None:
        out = torch.empty((B, N, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((B, N, Hq), dtype=torch.float32, device=q.device)
    _dev(out, "out", torch.float32, (B, N, Hq, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, N, Hq))
    need = attn_tree_workspace_bytes(B, N, Hq, Hkv, D, Tcap, window)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _dev(workspace, "workspace", torch.uint8)
    _check(lib().attn_tree_verify(B, N, Hq, Hkv, D, Tcap, KV_TYPES[k_type], KV_TYPES[v_type], int(window),
                                  float(scale), _ptr(parent), _ptr(n_nodes), _ptr(n_past), _ptr(q), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  _stream(q.device)))
    return out, lse


def attn_tree_verify_noalloc(q, k_cache, v_cache, k_type: str, v_type: str, n_past, parent, n_nodes, window: int,
                             scale: float, out, lse=None):
    """``attn_tree_verify`` without a workspace argument: the library's built-in scratch holds
    the split partials, so the call allocates nothing on the device.  ``out`` (and ``lse``, if
    wanted) must be passed in.  Calls that can overlap on one GPU race on the scratch."""
    B, N, Hq, D = q.shape
    Hkv, Tcap = k_cache.shape[1], k_cache.shape[2]
    _dev(q, "q", torch.bfloat16)
    _dev(k_cache, "k_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[k_type]))
    _dev(v_cache, "v_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[v_type]))
    _dev(n_past, "n_past", torch.int32, (B,))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    _dev(out, "out", torch.float32, (B, N, Hq, D))
    if lse is not None:
        _dev(lse, "lse", torch.float32, (B, N, Hq))
    _check(lib().attn_tree_verify_noalloc(B, N, Hq, Hkv, D, Tcap, KV_TYPES[k_type], KV_TYPES[v_type], int(window),
                                          float(scale), _ptr(parent), _ptr(n_nodes), _ptr(n_past), _ptr(q),
                                          _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(lse), _stream(q.device)))
    return out, lse


def tree_accept_workspace_bytes(B: int, N: int, V: int, dtype=torch.bfloat16) -> int:
    return int(lib().tree_accept_workspace_bytes(B, N, V, _in_dtype(torch.empty(0, dtype=dtype))))


def tree_accept_greedy(logits, parent, n_nodes, tokens, target=None, path=None, path_len=None,
                       next_token=None, workspace=None):
    """Greedy acceptance from the target's logits (bf16 or fp32 ``[B][N][V]``).  Returns
    ``(target, path, path_len, next_token)``: int32 ``[B][N]``, ``[B][N]``, ``[B]``, ``[B]``."""
    B, N, V = logits.shape
    _dev(logits, "logits", (torch.bfloat16, torch.float32))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    _dev(tokens, "tokens", torch.int32, (B, N))
    dev = logits.device
    target = torch.empty((B, N), dtype=torch.int32, device=dev) if target is None else target
    path = torch.empty((B, N), dtype=torch.int32, device=dev) if path is None else path
    path_len = torch.empty((B,), dtype=torch.int32, device=dev) if path_len is None else path_len
    next_token = torch.empty((B,), dtype=torch.int32, device=dev) if next_token is None else next_token
    _dev(target, "target", torch.int32, (B, N)); _dev(path, "path", torch.int32, (B, N))
    _dev(path_len, "path_len", torch.int32, (B,)); _dev(next_token, "next_token", torch.int32, (B,))
    if workspace is None:
        workspace = torch.empty(max(tree_accept_workspace_bytes(B, N, V, logits.dtype), 256), dtype=torch.uint8,
                                device=dev)
    _dev(workspace, "workspace", torch.uint8)
    _check(lib().tree_accept_greedy(B, N, V, _in_dtype(logits), _ptr(logits), _ptr(parent), _ptr(n_nodes),
                                    _ptr(tokens), _ptr(target), _ptr(path), _ptr(path_len), _ptr(next_token),
                                    _ptr(workspace), workspace.numel(), _stream(dev)))
    return target, path, path_len, next_token


def kv_tree_compact(k_cache, v_cache, k_type: str, v_type: str, n_past, path, path_len):
    """Move each sequence's accepted tree rows (slot n_past + path[m]) to slot n_past + m,
    in place, in both caches ``[B][Hkv][Tcap][row bytes]`` (uint8)."""
    B, Hkv, Tcap, rk = k_cache.shape
    D = rk // KV_BLOCK_BYTES[k_type] * 32
    _dev(k_cache, "k_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[k_type]))
    _dev(v_cache, "v_cache", torch.uint8, (B, Hkv, Tcap, D // 32 * KV_BLOCK_BYTES[v_type]))
    _dev(n_past, "n_past", torch.int32, (B,))
    _dev(path, "path", torch.int32); _dev(path_len, "path_len", torch.int32, (B,))
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError(f"path has shape {tuple(path.shape)}, expected ({B}, Lmax)")
    _check(lib().kv_tree_compact(B, Hkv, D, Tcap, KV_TYPES[k_type], KV_TYPES[v_type], _ptr(n_past), _ptr(path),
                                 _ptr(path_len), path.shape[1], _ptr(k_cache), _ptr(v_cache), _stream(k_cache.device)))
    return k_cache, v_cache


def conv_tree_verify(x, weight, conv_state, parent, n_nodes, activation: str = "none", y=None):
    """Tree-aware causal convolution.  x ``[B][N][C]`` (bf16 or fp32), weight fp32 ``[C][K]``,
    conv_state fp32 ``[B][K-1][C]`` (read only).  Returns y fp32 ``[B][N][C]``."""
    B, N, C = x.shape
    K = weight.shape[1]
    _dev(x, "x", (torch.bfloat16, torch.float32))
    _dev(weight, "weight", torch.float32, (C, K)); _dev(conv_state, "conv_state", torch.float32, (B, K - 1, C))
    _dev(parent, "parent", torch.int32, (B, N)); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    if y is None:
        y = torch.empty((B, N, C), dtype=torch.float32, device=x.device)
    _dev(y, "y", torch.float32, (B, N, C))
    _check(lib().conv_tree_verify(B, N, C, K, _in_dtype(x), ACTIVATIONS[activation], _ptr(parent), _ptr(n_nodes),
                                  _ptr(x), _ptr(weight), _ptr(conv_state), _ptr(y), _stream(x.device)))
    return y


def conv_tree_commit(conv_state, x, path, path_len):
    """Move the committed window (fp32 ``[B][K-1][C]``, in place) to the end of each
    sequence's accepted path."""
    B, Km1, C = conv_state.shape
    N = x.shape[1]
    _dev(conv_state, "conv_state", torch.float32)
    _dev(x, "x", (torch.bfloat16, torch.float32), (B, N, C))
    _dev(path, "path", torch.int32); _dev(path_len, "path_len", torch.int32, (B,))
    if path.dim() != 2 or path.shape[0] != B:
        raise ValueError(f"path has shape {tuple(path.shape)}, expected ({B}, Lmax)")
    _check(lib().conv_tree_commit(B, N, C, Km1 + 1, _in_dtype(x), _ptr(path), _ptr(path_len), path.shape[1],
                                  _ptr(x), _ptr(conv_state), _stream(x.device)))
    return conv_state


META_BITS = {"n_nodes": 1, "root": 2, "parent": 4, "path_len": 8, "path_root": 16, "path_step": 32}


def check_metadata(parent, n_nodes, path=None, path_len=None, status=None):
    """Device-side check of tree (and path) metadata; returns an int32 ``[B]`` device tensor of
    bit masks (``META_BITS``), 0 for a valid sequence.  Nothing is read back."""
    B, N = parent.shape
    _dev(parent, "parent", torch.int32); _dev(n_nodes, "n_nodes", torch.int32, (B,))
    Lmax = 1
    if path is not None or path_len is not None:
        _dev(path, "path", torch.int32); _dev(path_len, "path_len", torch.int32, (B,))
        if path.dim() != 2 or path.shape[0] != B:
            raise ValueError(f"path has shape {tuple(path.shape)}, expected ({B}, Lmax)")
        Lmax = path.shape[1]
    if status is None:
        status = torch.empty((B,), dtype=torch.int32, device=parent.device)
    _dev(status, "status", torch.int32, (B,))
    _check(lib().tv_check_metadata(_ptr(parent), _ptr(n_nodes), _ptr(path) if path is not None else None,
                                   _ptr(path_len) if path_len is not None else None, B, N, Lmax, _ptr(status),
                                   _stream(parent.device)))
    return status


def _host_i32(a, name):
    t = torch.as_tensor(a, dtype=torch.int32).contiguous()
    if t.device.type != "cpu":
        raise ValueError(f"{name} must be a host array for validation")
    return t


def validate_tree(parent, n_nodes) -> None:
    """Exact host-side check of tree metadata; raises TreeVerifyError (TV_ETOPO, ...)."""
    p, n = _host_i32(parent, "parent"), _host_i32(n_nodes, "n_nodes")
    B, N = p.shape
    _check(lib().tv_validate_tree(_ptr(p), _ptr(n), B, N))


def validate_path(parent, n_nodes, path, path_len) -> None:
    p, n = _host_i32(parent, "parent"), _host_i32(n_nodes, "n_nodes")
    a, L = _host_i32(path, "path"), _host_i32(path_len, "path_len")
    B, N = p.shape
    _check(lib().tv_validate_path(_ptr(p), _ptr(n), _ptr(a), _ptr(L), B, N, a.shape[1]))

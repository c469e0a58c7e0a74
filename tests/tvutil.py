"""Shared helpers for the parity tests: moving seeded inputs to the device and comparing."""
from __future__ import annotations

import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def t_bits(a: np.ndarray, device=None) -> torch.Tensor:
    """uint16 bf16 bit patterns -> torch.bfloat16 on the device."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device or dev())


def t_f32(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device or dev())


def t_i32(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device or dev())


def t_u8(a: np.ndarray, device=None) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(device or dev())


def lin_to_device(L):
    conv = t_bits if L.dtype == "bf16" else t_f32
    return dict(q=conv(L.q), k=conv(L.k), v=conv(L.v), g=conv(L.g), beta=conv(L.beta), state=t_f32(L.state),
                parent=t_i32(L.parent), n_nodes=t_i32(L.n_nodes), path=t_i32(L.path), path_len=t_i32(L.path_len))


def attn_to_device(A):
    return dict(q=t_bits(A.q), k_cache=t_u8(A.k_cache), v_cache=t_u8(A.v_cache), n_past=t_i32(A.n_past),
                parent=t_i32(A.parent), n_nodes=t_i32(A.n_nodes))


def rel_err(got, ref, mask=None) -> float:
    """max |got - ref| / RMS(ref), over the rows selected by ``mask`` (all if None)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        got, ref = got[mask], ref[mask]
    rms = float(np.sqrt(np.mean(ref ** 2)))
    return float(np.max(np.abs(got - ref))) / rms if rms > 0 else float(np.max(np.abs(got - ref)))


def valid_rows(n_nodes: np.ndarray, N: int) -> np.ndarray:
    """Boolean [B][N] mask of the rows that belong to each sequence's tree."""
    return np.arange(N)[None, :] < np.asarray(n_nodes)[:, None]

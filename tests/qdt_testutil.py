"""Helpers shared by the tests: host/device transfer of bf16 bit patterns and ulp distances."""
from __future__ import annotations

import numpy as np


def bf16_key(u) -> np.ndarray:
    """Order-preserving integer of a bf16 bit pattern (+0 and -0 map to the same key)."""
    u = np.asarray(u).astype(np.int64)
    return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + (u & 0x7FFF))


def ulp_bf16(a, b) -> np.ndarray:
    return np.abs(bf16_key(a) - bf16_key(b))


def is_nan_bf16(u) -> np.ndarray:
    u = np.asarray(u).astype(np.int64)
    return ((u & 0x7F80) == 0x7F80) & ((u & 0x7F) != 0)


def to_dev(a: np.ndarray, dev="cuda"):
    """numpy array -> torch device tensor; uint16 arrays become bfloat16 (same bits)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def to_host(t) -> np.ndarray:
    """torch tensor -> numpy; bfloat16 becomes uint16 bit patterns."""
    import torch
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bits_equal(a: np.ndarray, b: np.ndarray) -> bool:
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and tail rows plus a seeded sample, sorted and unique."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, M - 1, M - 2, M // 2]
    tail = list(range(max(0, M - (M % 256 or 256)), M))[:8]
    rows = np.unique(np.clip(np.concatenate([fixed, tail, rng.integers(0, M, n)]), 0, M - 1))
    return rows.astype(np.int64)


# Block-scaled FP4 exponents as the library stores them: stage-major [K/256, rows, 8], block 8 s + w
# of a row at byte MX_POS[w] of its 8-byte slot in stage s.  The oracle keeps them row-major
# [rows, K/32]; these two permutations convert between the layouts (no arithmetic).
MX_POS = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def mx_exponents_to_rows(S) -> np.ndarray:
    """[K/256, rows, 8] (library) -> [rows, K/32] (oracle)."""
    s = np.asarray(S)
    st, rows, _ = s.shape
    return np.ascontiguousarray(s[:, :, MX_POS].transpose(1, 0, 2).reshape(rows, st * 8))


def mx_exponents_from_rows(S) -> np.ndarray:
    """[rows, K/32] (oracle) -> [K/256, rows, 8] (library)."""
    s = np.asarray(S)
    rows, nb = s.shape
    out = np.empty((nb // 8, rows, 8), s.dtype)
    out[:, :, MX_POS] = s.reshape(rows, nb // 8, 8).transpose(1, 0, 2)
    return out

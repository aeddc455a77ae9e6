"""Helpers for the GPU parity tests: device buffers from numpy bits and back."""

from __future__ import annotations

import sys

import numpy as np


def torch():
    import torch as _t
    return _t


def dev(arr: np.ndarray):
    """numpy -> device tensor with the same bytes (uint16 kept as int16 bits)."""
    t = torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return t.from_numpy(a).to("cuda")


def host(t, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def zeros_u16(*shape):
    t = torch()
    return t.zeros(*shape, dtype=t.int16, device="cuda")


def zeros_f32(*shape):
    t = torch()
    return t.zeros(*shape, dtype=t.float32, device="cuda")


def zeros_bytes(n):
    t = torch()
    return t.zeros(max(n, 16), dtype=t.uint8, device="cuda")


def say(*args):
    """Prints and flushes at once, so that a case is named before its GPU step."""
    print(*args, flush=True)
    sys.stdout.flush()


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got.astype(np.float64) - ref))) if got.size else 0.0

"""Exact widening of cache-dtype inputs to float64, and narrowing of results.

bf16 arrays arrive as their uint16 bit patterns (numpy has no bf16 type); a
bf16 value is the float32 whose upper 16 bits are those bits, so widening is
exact. Narrowing (used only for ZIP-merged rows, which the cache stores in
its own dtype) rounds to nearest, ties to even.
"""
from __future__ import annotations

import numpy as np


def to_f64(x, dtype: str | None = None) -> np.ndarray:
    """Widen bf16 bit patterns (uint16/int16) or a float array to float64, exactly."""
    a = np.asarray(x)
    if dtype == "bf16" or a.dtype in (np.uint16, np.int16):
        bits = a.view(np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_f32(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16): first to float32 (RNE), then the
    float32 bits to bf16 by round-to-nearest-even on the dropped 16 bits."""
    f = round_to_f32(x)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)

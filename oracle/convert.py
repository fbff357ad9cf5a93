"""Exact widening of cache-dtype inputs to float64, and narrowing of results.

TEST INFRASTRUCTURE (part of the CPU oracle; the product path never imports it).

bf16 arrays arrive as their uint16 bit patterns (numpy has no bf16 type); a
bf16 value is the float32 whose upper 16 bits are those bits, so widening is
exact. Narrowing (used only for ZIP-merged rows, which the cache stores in
its own dtype; reading R13: the merged row is rounded to nearest, ties to
even, from its exact value) is a single rounding of the float64 value.
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
    """float64 -> float32, round to nearest, ties to even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def _f32_round_to_odd(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 bits rounded to odd: truncate toward zero, then set the
    last bit if anything was dropped. A later round-to-nearest-even that drops
    at least two more bits then equals one rounding of the float64 value."""
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    away = np.abs(f.astype(np.float64)) > np.abs(x)          # nearest rounding went away from zero
    f = np.where(away, np.nextafter(f, np.float32(0)), f)
    u = f.view(np.uint32).copy()
    inexact = f.astype(np.float64) != x
    u[inexact] |= np.uint32(1)
    return u


def round_to_bf16(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), one rounding to nearest, ties to
    even: float32 bits rounded to odd (so no tie is created by the first step),
    then round-to-nearest-even on the 16 dropped bits."""
    u = _f32_round_to_odd(x).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)

"""Choosing the tokens to evict.

InertiaKV §3.1: when the cache exceeds the budget B, evict the tokens with the
lowest utility m_t(i). MomentKV Algorithm 1, phase 1, does the same one token
at a time: while |R| > L, take the argmin of the score, remove it, repeat.

The pages never say how exact ties are broken. Reading used here: the order
is (value, position) ascending, so among equal values the older token (lower
position) goes first. That makes every selection unique.

LaProx notes, key design 3: a model-wide Top-K over every (layer, head,
token) score keeps the K largest; that is the same order with the bottom
n - K evicted, ties broken by the flat index.
"""
from __future__ import annotations

import numpy as np


def bottom_k(values, pos, k: int) -> np.ndarray:
    """Slot indices (sorted) of the k smallest entries under (value, pos) ascending."""
    values = np.asarray(values, dtype=np.float64)
    pos = np.asarray(pos)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((pos, values))      # primary key: value, secondary: pos
    return np.sort(order[:k]).astype(np.int64)


def bottom_k_protected(values, pos, k: int, protect_from) -> np.ndarray:
    """Slot indices (sorted) of the k smallest entries under (protected, value, pos)
    ascending, protected meaning pos >= protect_from: InertiaKV §3.1's third lazy-refresh
    alternative, where entries not yet scored are kept while others can go."""
    values = np.asarray(values, dtype=np.float64)
    pos = np.asarray(pos)
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((pos, values, pos >= protect_from))
    return np.sort(order[:k]).astype(np.int64)


def bottom_k_one_at_a_time(values, pos, k: int) -> np.ndarray:
    """MomentKV Algorithm 1 phase 1 with a score that does not depend on the
    evicted set: repeatedly remove the minimum (ties to the lower position)."""
    values = list(np.asarray(values, dtype=np.float64))
    pos = list(np.asarray(pos))
    live = list(range(len(values)))
    out = []
    for _ in range(max(0, k)):
        best = live[0]
        for j in live[1:]:
            if values[j] < values[best] or (values[j] == values[best] and pos[j] < pos[best]):
                best = j
        out.append(best)
        live.remove(best)
    return np.sort(np.array(out, dtype=np.int64))


def top_k_keep(scores, K: int) -> np.ndarray:
    """Boolean keep mask of the K largest scores (flat), by evicting the
    bottom n - K under (score, flat index) ascending."""
    s = np.asarray(scores, dtype=np.float64).ravel()
    keep = np.ones(s.size, dtype=bool)
    keep[bottom_k(s, np.arange(s.size), s.size - K)] = False
    return keep.reshape(np.shape(scores))

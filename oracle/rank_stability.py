"""Rank-stability diagnostic (test infrastructure).

InertiaKV §3.1 measures how stable a scorer's ranking is by the Jaccard similarity of the
token sets two scorers (or two steps) keep (Fig. 1: about 0.97 between scorers under EMA
aggregation). Written out with Python sets: |A and B| / |A or B|, 1 for two empty sets.
"""
from __future__ import annotations

import numpy as np


def keep_jaccard(keep_a, keep_b) -> float:
    A = set(np.flatnonzero(np.asarray(keep_a)).tolist())
    B = set(np.flatnonzero(np.asarray(keep_b)).tolist())
    union = A | B
    return 1.0 if not union else len(A & B) / len(union)

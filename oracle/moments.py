"""MomentKV moment statistics of the evicted tokens.

MomentKV §4.1 (efficient statistics update) and Appendix A.1: the evicted set
is summarised by four running sums, each updated by one addition per evicted
token and never revisited:
  n_e  count,  s_k = sum k_i,  s_v = sum v_i,  S = sum v_i k_i^T  (d x d).
Algorithm 1, steps 11-13, adds them in the order tokens are evicted. The
centred view used by the first-order estimate is k_bar = s_k/n_e,
v_bar = s_v/n_e and S_tilde = S - s_v s_k^T / n_e.
"""
from __future__ import annotations

import numpy as np


def empty_moments(n_units: int, d: int) -> dict:
    """Statistics at the start of generation: all zero (MomentKV, experimental setup)."""
    return {"n": 0, "sk": np.zeros((n_units, d)), "sv": np.zeros((n_units, d)),
            "S": np.zeros((n_units, d, d))}


def fold_moments(mom: dict, K_E, V_E) -> dict:
    """Fold evicted rows into the statistics of every unit of a scope.

    mom: {"n": int, "sk": [U, d], "sv": [U, d], "S": [U, d, d]} (float64);
    K_E, V_E: [U, k, d] evicted rows. S[u][a][b] += sum_e v_{e,a} k_{e,b}.
    """
    K_E = np.asarray(K_E, dtype=np.float64)
    V_E = np.asarray(V_E, dtype=np.float64)
    k = K_E.shape[1]
    S = mom["S"].copy()
    for u in range(K_E.shape[0]):
        S[u] += V_E[u].T @ K_E[u]          # sum_e v_e k_e^T as one matmul
    return {"n": mom["n"] + k, "sk": mom["sk"] + K_E.sum(axis=1), "sv": mom["sv"] + V_E.sum(axis=1), "S": S}


def centred_moments(mom: dict):
    """(k_bar [U,d], v_bar [U,d], S_tilde [U,d,d]) from the running sums; n_e must be > 0."""
    n = float(mom["n"])
    kbar = mom["sk"] / n
    vbar = mom["sv"] / n
    St = mom["S"] - np.einsum("ua,ub->uab", mom["sv"], mom["sk"]) / n
    return kbar, vbar, St

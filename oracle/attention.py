"""Vote-weighted decode attention of one KV head and the head-averaged score.

KeepKV notes, eq. (1): o = sum_i s_i v_i / sum_i s_i with the unnormalised
score s_i = exp(q.k_i / sqrt(d)). Eq. (6) (restated as eq. (23)) gives every
entry an integer vote p_i: o = sum_i p_i s_i v_i / sum_i p_i s_i; all votes
equal to 1 is eq. (22), plain attention. The integration notes implement the
vote by adding ln p_i to the logit before the softmax, i.e. the per-token
weight a_i = p_i s_i / sum_j p_j s_j.

InertiaKV §3.1, eq. (1): s_t(i) = (1/H) sum_h a_t^(h)(i), the last-query
attention weights averaged over heads.
"""
from __future__ import annotations

import numpy as np


def attend_unit(q, K, V, votes, scale):
    """One KV head with G query heads.

    q [G, d], K [L, d], V [L, d] float64; votes [L] (None means all ones);
    scale = tau (1/sqrt(d) unless the caller says otherwise).

    Returns (logits [G, L], a [G, L], o [G, d], lse [G]) where
      logits_{g,i} = tau * q_g . k_i
      a_{g,i}      = p_i exp(logits_{g,i}) / Z_g,  Z_g = sum_i p_i exp(logits_{g,i})
      o_g          = sum_i a_{g,i} v_i
      lse_g        = ln Z_g
    The exponentials are evaluated as exp(logit - max_i logit) and the max
    added back into lse (shift invariance of the ratio). With no live token,
    or every vote zero, Z = 0: then a = 0, o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    G, d = q.shape
    L = K.shape[0]
    p = np.ones(L) if votes is None else np.asarray(votes, dtype=np.float64)
    logits = scale * (q @ K.T)
    if L == 0:
        return logits, np.zeros((G, 0)), np.zeros((G, d)), np.full(G, -np.inf)
    M = logits.max(axis=1, keepdims=True)
    w = p[None, :] * np.exp(logits - M)
    Z = w.sum(axis=1, keepdims=True)
    safe = np.where(Z > 0, Z, 1.0)
    a = np.where(Z > 0, w / safe, 0.0)
    o = a @ V
    with np.errstate(divide="ignore"):
        lse = M[:, 0] + np.log(Z[:, 0])
    return logits, a, o, lse


def scope_score(a_per_unit):
    """s(i) = mean of a_{g,i} over every query head of every unit in the scope.
    a_per_unit: list of [G, L] arrays sharing the slot axis."""
    A = np.concatenate([np.asarray(a, dtype=np.float64) for a in a_per_unit], axis=0)
    return A.mean(axis=0)

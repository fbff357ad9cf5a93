"""MomentKV moment-informed eviction (test infrastructure, fp64).

MomentKV summary page, §4.2 ("moment residual", "moment-aware eviction
score") and Algorithm 1 phase 1. For one attention head, the evicted set E is
known only through its running sums (n_e, s_k, s_v, S) (§4.1). Each retained
token j is compared with the affine model those sums define, evaluated at its
own key:

  if n_e > 0:  k_bar = s_k / n_e,  v_bar = s_v / n_e,  S_tilde = S - s_v s_k^T / n_e,
               r_j = v_j - v_bar - tau S_tilde (k_j - k_bar) / n_e;
  if n_e = 0:  v_bar and S_tilde are zero, so r_j = v_j;
  score(j) = alpha_j ||r_j||_2,

with alpha the softmax attention weights over the retained set and tau the
softmax scale (the page's 1/sqrt(d)). While the retained set holds more than
the budget, the token of lowest score is evicted, folded into the sums
(n_e += 1, s_k += k, s_v += v, S += v k^T) and removed; the next eviction is
scored with the updated sums and alpha renormalised over what is left.

Readings (the page leaves these open):
  * under GQA the head is a KV head, and alpha is the mean over its query heads
    of their softmax weights (the head-averaged weight s(i) of the step);
  * equal scores go to the lower position first (as every selection here);
  * renormalising alpha scales every remaining score by the same factor, so it
    is done literally below but cannot change which token is lowest.
"""
from __future__ import annotations

import numpy as np


def moment_residuals(K, V, mom_unit, scale):
    """r [L, d]: each row's value minus the moment model's prediction at its key.

    K, V [L, d]; mom_unit = {"n", "sk" [d], "sv" [d], "S" [d, d]} with
    S[a][b] = sum_e v_{e,a} k_{e,b}."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n = float(mom_unit["n"])
    if n == 0:
        return V.copy()
    sk = np.asarray(mom_unit["sk"], dtype=np.float64)
    sv = np.asarray(mom_unit["sv"], dtype=np.float64)
    S = np.asarray(mom_unit["S"], dtype=np.float64)
    k_bar = sk / n
    v_bar = sv / n
    S_tilde = S - np.outer(sv, sk) / n
    # (S_tilde (k_j - k_bar))_a = sum_b S_tilde[a][b] (k_j - k_bar)_b, for every row j at once
    pred = v_bar[None, :] + scale * ((K - k_bar[None, :]) @ S_tilde.T) / n
    return V - pred


def moment_scores(K, V, alpha, mom_unit, scale, live=None):
    """score(j) = alpha_j ||r_j|| over the live rows (alpha renormalised over them);
    rows that are not live get +inf."""
    alpha = np.asarray(alpha, dtype=np.float64)
    L = alpha.shape[0]
    live = np.ones(L, dtype=bool) if live is None else np.asarray(live, dtype=bool)
    total = alpha[live].sum()
    a = alpha / total if total > 0 else alpha
    r = moment_residuals(K, V, mom_unit, scale)
    norms = np.sqrt((r * r).sum(axis=1))
    return np.where(live, a * norms, np.inf)


def fold_one(mom_unit, k, v):
    """Algorithm 1 steps 11-13 for one evicted token (float64 sums)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    return {"n": mom_unit["n"] + 1, "sk": mom_unit["sk"] + k, "sv": mom_unit["sv"] + v,
            "S": mom_unit["S"] + np.outer(v, k)}


def lowest(scores, pos, live):
    """Index of the lowest live score, ties to the lower position."""
    cand = np.flatnonzero(live)
    order = np.lexsort((np.asarray(pos)[cand], np.asarray(scores)[cand]))
    return int(cand[order[0]])


def moment_informed_evict(K, V, alpha, pos, mom_unit, budget, scale, choose=None):
    """Algorithm 1 phase 1 on one head whose retained set is rows [0, L).

    Returns (order, mom_after, first_scores, scores_per_step): the evicted rows
    in eviction order, the sums after folding them, the scores of the first
    round (every row live) and the scores of every round. `choose(step, scores,
    live)` may return the row to evict in place of the lowest one (a test
    follows another implementation's pick through near-ties with it); by
    default the lowest score is taken."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    L = K.shape[0]
    live = np.ones(L, dtype=bool)
    mom = {"n": int(mom_unit["n"]), "sk": np.array(mom_unit["sk"], dtype=np.float64),
           "sv": np.array(mom_unit["sv"], dtype=np.float64), "S": np.array(mom_unit["S"], dtype=np.float64)}
    order, rounds = [], []
    first = moment_scores(K, V, alpha, mom, scale, live)
    step = 0
    while live.sum() > budget:
        sc = first if step == 0 else moment_scores(K, V, alpha, mom, scale, live)
        rounds.append(sc)
        j = lowest(sc, pos, live) if choose is None else int(choose(step, sc, live))
        mom = fold_one(mom, K[j], V[j])
        live[j] = False
        order.append(j)
        step += 1
    return np.array(order, dtype=np.int64), mom, first, rounds

"""KeepKV ZIP-merging of an evicted entry into a partner entry.

KeepKV notes:
  * candidate choice: merge pairs are chosen by the cosine similarity of
    their keys ("why cosine similarity"); here the partner c of the evicted e
    is the live entry with the largest cos(k_e, k_c), ties to the lower
    position, no recent-token exclusion (the page leaves R open).
  * eq. (7): the merged entry's vote is p_r = p_e + p_c.
  * eqs. (8)-(10): with w_x = p_x s_x, v_r = (w_e v_e + w_c v_c) / (w_e + w_c).
  * eq. (12) (= eq. (21)):
        k_r = (w_e k_e + w_c k_c) ln((w_e + w_c)/(p_e + p_c)) / (w_e ln s_e + w_c ln s_c)
    where ln s_x is the logit itself ("numerical stability", item 1).
  * "numerical stability", item 2: if |w_e ln s_e + w_c ln s_c| < eps, fall
    back to k_r = (k_e + k_c)/2.

Readings: the pages treat one query head (MHA). Under GQA the reference
logit is the group-mean logit lbar_i = mean_g logit_{g,i}, which is exactly
the logit of the group-mean query; the merge is then lossless for that query.

Evaluation: with mu = max(lbar_e, lbar_c) and hat-w_x = p_x exp(lbar_x - mu)
(w_x = hat-w_x e^mu), eq. (12) becomes
    k_r = (hat-w_e k_e + hat-w_c k_c) * Num / Den,
    Num = mu + ln(hat-w_e + hat-w_c) - ln(p_e + p_c),
    Den = hat-w_e lbar_e + hat-w_c lbar_c,
and the page's guard |w_e ln s_e + w_c ln s_c| < eps reads |Den| < eps e^{-mu}.
"""
from __future__ import annotations

import numpy as np


def cosine_partner(K, e: int, pos) -> int:
    """argmax over j != e of cos(k_e, k_j); ties to the lower position.
    A zero-norm key has cosine 0 with everything."""
    K = np.asarray(K, dtype=np.float64)
    pos = np.asarray(pos)
    nrm = np.sqrt((K * K).sum(axis=1))
    dots = K @ K[e]
    denom = nrm * nrm[e]
    cos = np.where(denom > 0, dots / np.where(denom > 0, denom, 1.0), 0.0)
    best = -1
    for j in range(K.shape[0]):
        if j == e:
            continue
        if best < 0 or cos[j] > cos[best] or (cos[j] == cos[best] and pos[j] < pos[best]):
            best = j
    return best


def zip_merge(k_e, v_e, p_e, lbar_e, k_c, v_c, p_c, lbar_c, eps: float = 1e-6):
    """Returns (k_r, v_r, p_r, guarded) in float64."""
    k_e, v_e, k_c, v_c = (np.asarray(x, dtype=np.float64) for x in (k_e, v_e, k_c, v_c))
    p_e, p_c = float(p_e), float(p_c)
    mu = max(lbar_e, lbar_c)
    we = p_e * np.exp(lbar_e - mu)
    wc = p_c * np.exp(lbar_c - mu)
    v_r = (we * v_e + wc * v_c) / (we + wc)
    num = mu + np.log(we + wc) - np.log(p_e + p_c)
    den = we * lbar_e + wc * lbar_c
    guarded = abs(den) < eps * np.exp(-mu)
    if guarded:
        k_r = 0.5 * (k_e + k_c)
    else:
        k_r = (we * k_e + wc * k_c) * (num / den)
    return k_r, v_r, int(p_e + p_c), bool(guarded)

"""KeepKV prefill compression by greedy all-pairs ZIP merging (test infrastructure, fp64).

KeepKV reading notes, the inference algorithm's prefill steps 2-5 and the
paragraphs on candidate choice: every entry starts with vote 1; while the
cache holds more than B entries, the pair of entries whose keys have the
largest cosine similarity, both outside the most recent tokens, is merged
(eqs. (7), (10), (12) with the numerical-stability guard) using the exact
attention scores of the prefill's last query, and the pair is replaced by the
merged entry.

Readings (the notes leave these open):
  * the reference score of an entry is the group-mean logit under GQA (the
    logit of the group-mean query), as for the decode-time merge; a merged
    entry's score for later merges is its own logit, recomputed from its
    merged key (without the guard this is ln((w_e + w_c)/(p_e + p_c)));
  * "the most recent R tokens" are given as a position bound: entries at
    positions >= protect_from never merge;
  * the merged entry keeps the slot and position of the older of the two and
    the sum of their utilities; its rows are rounded to the cache dtype;
  * ties: cosine descending, then the pair's lower position, then its higher
    position; a zero key has cosine 0 with everything.
"""
from __future__ import annotations

import numpy as np

from .convert import round_to_bf16, round_to_f32, to_f64
from .zip_merge import zip_merge


def _round_rows(x, row_dtype):
    if row_dtype == "bf16":
        return to_f64(round_to_bf16(x), "bf16")
    if row_dtype == "f32":
        return round_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def reference_logits(K, q, scale):
    """lbar_i = mean over the G query heads of scale * q_g . k_i."""
    q = np.asarray(q, dtype=np.float64).reshape(-1, np.asarray(K).shape[-1])
    return scale * (np.asarray(K, dtype=np.float64) @ q.T).mean(axis=1)


def cosine_matrix(K):
    K = np.asarray(K, dtype=np.float64)
    n = np.sqrt((K * K).sum(axis=1))
    den = np.outer(n, n)
    dots = K @ K.T
    return np.where(den > 0, dots / np.where(den > 0, den, 1.0), 0.0)


def best_pair(K, pos, cand):
    """(i, j, cos) of the candidate pair of largest cosine; ties to the lower (min pos, max pos)."""
    idx = np.flatnonzero(cand)
    if idx.size < 2:
        return None
    C = cosine_matrix(np.asarray(K)[idx])
    iu, ju = np.triu_indices(idx.size, k=1)
    c = C[iu, ju]
    top = np.flatnonzero(c == c.max())
    p = np.asarray(pos)[idx]
    lo = np.minimum(p[iu[top]], p[ju[top]])
    hi = np.maximum(p[iu[top]], p[ju[top]])
    t = top[np.lexsort((hi, lo))[0]]
    return int(idx[iu[t]]), int(idx[ju[t]]), float(c[t])


def prefill_merge(K, V, votes, pos, m, q, scale, budget, protect_from, eps=1e-6, row_dtype="f64",
                  choose=None):
    """Greedy prefill merging of one head's entries [0, L).

    Returns a dict with the final K, V, votes, m (arrays over the original
    slots; merged-away slots keep stale rows), the live mask, the merge
    sequence [(survivor, removed), ...] and whether any merge was guarded.
    `choose(step, K, cand)` may return the pair to merge in place of the best
    one (a test follows another implementation through near-ties)."""
    K = np.array(K, dtype=np.float64)
    V = np.array(V, dtype=np.float64)
    votes = np.array(votes, dtype=np.int64)
    pos = np.asarray(pos)
    m = np.array(m, dtype=np.float64)
    L = K.shape[0]
    live = np.ones(L, dtype=bool)
    cand = pos < protect_from
    seq, guarded_any, step = [], False, 0
    while live.sum() > budget:
        if choose is not None:
            pair = choose(step, K, live & cand)
        else:
            bp = best_pair(K, pos, live & cand)
            pair = None if bp is None else bp[:2]
        if pair is None:
            break
        i, j = int(pair[0]), int(pair[1])
        surv, gone = (i, j) if pos[i] < pos[j] else (j, i)
        lb = reference_logits(K[[gone, surv]], q, scale)
        k_r, v_r, p_r, guarded = zip_merge(K[gone], V[gone], votes[gone], lb[0],
                                           K[surv], V[surv], votes[surv], lb[1], eps)
        guarded_any |= guarded
        K[surv] = _round_rows(k_r, row_dtype)
        V[surv] = _round_rows(v_r, row_dtype)
        votes[surv] = p_r
        m[surv] = m[surv] + m[gone]
        live[gone] = False
        seq.append((surv, gone))
        step += 1
    return {"K": K, "V": V, "votes": votes, "m": m, "live": live, "pairs": seq, "guarded": guarded_any}

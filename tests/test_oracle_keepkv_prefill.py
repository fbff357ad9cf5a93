"""Pins of the oracle's KeepKV prefill compression by greedy all-pairs ZIP merging (CPU only).

Tied to things other than the loop itself:
  * KeepKV's lossless property (each merge is exact for the query whose scores
    it uses): with rows kept in float64 and no guarded merge, attention of the
    reference query over the compressed cache, votes included, equals attention
    over the full prompt -- textbook attention of attend_unit, pinned to torch
    elsewhere; under GQA the same holds for the group-mean query;
  * votes sum to the prompt length; protected positions are untouched;
  * the pair taken is the brute-force maximum cosine written out in plain Python,
    in the first round and after a merge changed a key; equal keys tie to the
    lower positions.
"""
import math

import numpy as np

from oracle import attend_unit
from oracle.keepkv_prefill import prefill_merge, reference_logits

RNG = np.random.default_rng(11)
D = 16
TAU = 1.0 / math.sqrt(D)


def _prompt(L, spread=1.0):
    K = spread * RNG.standard_normal((L, D))
    V = RNG.standard_normal((L, D))
    return K, V, np.ones(L, dtype=np.int64), np.arange(L), np.zeros(L)


def _compressed(res):
    live = res["live"]
    return res["K"][live], res["V"][live], res["votes"][live]


def test_lossless_for_the_reference_query():
    L, B = 28, 9
    K, V, votes, pos, m = _prompt(L)
    q = RNG.standard_normal((1, D))
    res = prefill_merge(K, V, votes, pos, m, q, TAU, B, protect_from=L - 3)
    assert not res["guarded"] and res["live"].sum() == B
    Kc, Vc, pc = _compressed(res)
    _, _, o_full, lse_full = attend_unit(q, K, V, None, TAU)
    _, _, o_c, lse_c = attend_unit(q, Kc, Vc, pc, TAU)
    np.testing.assert_allclose(o_c, o_full, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse_c, lse_full, rtol=0, atol=1e-10)
    # another query is not reproduced (the merge is exact for the reference query only)
    q2 = RNG.standard_normal((1, D))
    assert np.abs(attend_unit(q2, Kc, Vc, pc, TAU)[2] - attend_unit(q2, K, V, None, TAU)[2]).max() > 1e-6


def test_lossless_for_the_group_mean_query_under_gqa():
    L, B, G = 24, 8, 4
    K, V, votes, pos, m = _prompt(L)
    q = RNG.standard_normal((G, D))
    res = prefill_merge(K, V, votes, pos, m, q, TAU, B, protect_from=L)
    assert not res["guarded"]
    Kc, Vc, pc = _compressed(res)
    qbar = q.mean(axis=0, keepdims=True)
    np.testing.assert_allclose(attend_unit(qbar, Kc, Vc, pc, TAU)[2], attend_unit(qbar, K, V, None, TAU)[2],
                               rtol=0, atol=1e-10)


def test_votes_budget_and_protected_positions():
    L, B, R = 30, 12, 5
    K, V, votes, pos, m = _prompt(L)
    m = RNG.random(L)
    q = RNG.standard_normal((2, D))
    res = prefill_merge(K, V, votes, pos, m, q, TAU, B, protect_from=L - R, row_dtype="bf16")
    assert res["live"].sum() == B
    assert res["votes"][res["live"]].sum() == L
    np.testing.assert_allclose(res["m"][res["live"]].sum(), m.sum(), rtol=1e-12)
    prot = pos >= L - R
    assert res["live"][prot].all()
    assert np.array_equal(res["K"][prot], K[prot]) and np.array_equal(res["V"][prot], V[prot])
    assert (res["votes"][prot] == 1).all()
    for surv, gone in res["pairs"]:
        assert pos[surv] < pos[gone] and not prot[surv] and not prot[gone]


def _brute_pair(K, pos, cand):
    best = None
    idx = [i for i in range(len(pos)) if cand[i]]
    for a in range(len(idx)):
        for b in range(a + 1, len(idx)):
            i, j = idx[a], idx[b]
            dot = sum(K[i][t] * K[j][t] for t in range(D))
            ni = math.sqrt(sum(K[i][t] ** 2 for t in range(D)))
            nj = math.sqrt(sum(K[j][t] ** 2 for t in range(D)))
            c = dot / (ni * nj)
            key = (-c, min(pos[i], pos[j]), max(pos[i], pos[j]))
            if best is None or key < best[0]:
                best = (key, i, j)
    return {best[1], best[2]}


def test_pairs_are_the_brute_force_maximum_cosine_round_by_round():
    L, B = 14, 6
    K, V, votes, pos, m = _prompt(L)
    pos = RNG.permutation(L) + 100
    q = RNG.standard_normal((1, D))
    seen = []

    def follow(step, Kcur, cand):
        pair = _brute_pair(Kcur, pos, cand)
        seen.append(pair)
        return tuple(pair)

    res = prefill_merge(K, V, votes, pos, m, q, TAU, B, protect_from=10 ** 9, choose=follow)
    ref = prefill_merge(K, V, votes, pos, m, q, TAU, B, protect_from=10 ** 9)
    assert [set(p) for p in ref["pairs"]] == seen
    # at least one round merged an entry that an earlier round had produced
    survivors = set()
    chained = False
    for surv, gone in ref["pairs"]:
        chained |= surv in survivors or gone in survivors
        survivors.add(surv)
    assert chained


def test_equal_keys_tie_to_the_lower_positions():
    K, V, votes, pos, m = _prompt(8)
    K[5] = K[2]
    K[7] = K[2]          # cos = 1 for (2, 5), (2, 7), (5, 7)
    pos = np.array([0, 1, 2, 3, 4, 5, 6, 7])
    res = prefill_merge(K, V, votes, pos, m, RNG.standard_normal((1, D)), TAU, 7, protect_from=100)
    assert res["pairs"] == [(2, 5)]


def test_stops_when_too_few_entries_may_merge():
    K, V, votes, pos, m = _prompt(10)
    res = prefill_merge(K, V, votes, pos, m, RNG.standard_normal((1, D)), TAU, 2, protect_from=4)
    assert res["live"].sum() == 7 and len(res["pairs"]) == 3


def test_reference_logits_are_the_group_mean_query_logits():
    K = RNG.standard_normal((5, D))
    q = RNG.standard_normal((3, D))
    np.testing.assert_allclose(reference_logits(K, q, TAU), TAU * K @ q.mean(axis=0), rtol=1e-13)

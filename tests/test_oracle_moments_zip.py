"""Pins of the oracle's moment fold, ZIP merge and compaction (CPU only).

MomentKV §4.1, Appendix A.1, Appendix B; KeepKV eqs. (6)-(12), Theorem 3,
Figure 3 worked votes, "numerical stability" guard.
"""
import os

import numpy as np
import pytest

from oracle import (attend_unit, centred_moments, compact, cosine_partner, empty_moments,
                    fold_moments, zip_merge)

RNG = np.random.default_rng(7)
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_centred_covariance_identity():
    """S_tilde = S - s_v s_k^T / n equals sum_E v_i (k_i - k_bar)^T computed directly."""
    U, k, d = 2, 23, 8
    KE, VE = RNG.standard_normal((U, k, d)), RNG.standard_normal((U, k, d))
    mom = fold_moments(empty_moments(U, d), KE, VE)
    assert mom["n"] == k
    kbar, vbar, St = centred_moments(mom)
    for u in range(U):
        np.testing.assert_allclose(kbar[u], KE[u].mean(axis=0), rtol=1e-14)
        np.testing.assert_allclose(vbar[u], VE[u].mean(axis=0), rtol=1e-13, atol=1e-15)
        direct = sum(np.outer(VE[u, i], KE[u, i] - KE[u].mean(axis=0)) for i in range(k))
        np.testing.assert_allclose(St[u], direct, rtol=1e-11, atol=1e-12)


def test_fold_is_incremental_and_order_free():
    U, d = 1, 6
    KE, VE = RNG.standard_normal((U, 12, d)), RNG.standard_normal((U, 12, d))
    once = fold_moments(empty_moments(U, d), KE, VE)
    step = empty_moments(U, d)
    for i in RNG.permutation(12):           # one token at a time, any order
        step = fold_moments(step, KE[:, i:i + 1], VE[:, i:i + 1])
    assert step["n"] == once["n"] == 12
    for key in ("sk", "sv", "S"):
        np.testing.assert_allclose(step[key], once[key], rtol=1e-13, atol=1e-14)


def test_jensen_lower_bound_on_evicted_partition():
    """MomentKV Appendix B: n_e exp(q.k_bar / sqrt d) <= Z_E, with equality when every
    evicted key is equal. Checks that the stored sums carry what the bound needs."""
    d = 16
    q = RNG.standard_normal(d)
    KE = RNG.standard_normal((1, 30, d))
    mom = fold_moments(empty_moments(1, d), KE, RNG.standard_normal((1, 30, d)))
    kbar, _, _ = centred_moments(mom)
    tau = 1 / np.sqrt(d)
    ZE = np.exp(tau * KE[0] @ q).sum()
    assert mom["n"] * np.exp(tau * q @ kbar[0]) <= ZE
    same = np.repeat(KE[:, :1], 30, axis=1)
    mom2 = fold_moments(empty_moments(1, d), same, same)
    k2, _, _ = centred_moments(mom2)
    np.testing.assert_allclose(30 * np.exp(tau * q @ k2[0]), np.exp(tau * same[0] @ q).sum(), rtol=1e-13)


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split())
    return rows


def test_zip_worked_votes():
    """KeepKV Figure 3: (p_e = 1) merged into (p_c = 2) gives p_r = 3."""
    for pe, pc, pr in _read_table("keepkv_zip_worked_example.txt"):
        d = 8
        _, _, p_r, _ = zip_merge(RNG.standard_normal(d), RNG.standard_normal(d), int(pe), 0.3,
                                 RNG.standard_normal(d), RNG.standard_normal(d), int(pc), -0.2)
        assert p_r == int(pr)


@pytest.mark.parametrize("trial", range(10))
def test_zip_merge_is_lossless_for_the_reference_query(trial):
    """KeepKV Theorem 3: with eqs. (10) and (12) and vote-weighted attention (6), the
    output for the query the merge used is unchanged; eq. (8) p_r s_r = p_e s_e + p_c s_c."""
    L, d = 20, 16
    tau = 1 / np.sqrt(d)
    q = RNG.standard_normal((1, d))
    K, V = RNG.standard_normal((L, d)), RNG.standard_normal((L, d))
    votes = RNG.integers(1, 5, size=L)
    logits, _, o, lse = attend_unit(q, K, V, votes, tau)
    e, c = RNG.choice(L, size=2, replace=False)
    k_r, v_r, p_r, guarded = zip_merge(K[e], V[e], votes[e], logits[0, e], K[c], V[c], votes[c],
                                       logits[0, c])
    assert not guarded
    lhs = p_r * np.exp(tau * q[0] @ k_r)
    rhs = votes[e] * np.exp(logits[0, e]) + votes[c] * np.exp(logits[0, c])
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12)
    K2, V2, p2 = K.copy(), V.copy(), votes.copy()
    K2[c], V2[c], p2[c] = k_r, v_r, p_r
    keep = np.arange(L) != e
    _, _, o2, lse2 = attend_unit(q, K2[keep], V2[keep], p2[keep], tau)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, rtol=1e-12)


def test_zip_group_mean_query_is_lossless_under_gqa():
    """Reading for GQA: merging with the group-mean logit is lossless for the mean query."""
    G, L, d = 4, 15, 16
    tau = 1 / np.sqrt(d)
    q = RNG.standard_normal((G, d))
    K, V = RNG.standard_normal((L, d)), RNG.standard_normal((L, d))
    votes = RNG.integers(1, 4, size=L)
    logits, _, _, _ = attend_unit(q, K, V, votes, tau)
    lbar = logits.mean(axis=0)
    qbar = q.mean(axis=0, keepdims=True)
    _, _, obar, _ = attend_unit(qbar, K, V, votes, tau)
    e, c = 3, 9
    k_r, v_r, p_r, _ = zip_merge(K[e], V[e], votes[e], lbar[e], K[c], V[c], votes[c], lbar[c])
    K2, V2, p2 = K.copy(), V.copy(), votes.copy()
    K2[c], V2[c], p2[c] = k_r, v_r, p_r
    keep = np.arange(L) != e
    _, _, obar2, _ = attend_unit(qbar, K2[keep], V2[keep], p2[keep], tau)
    np.testing.assert_allclose(obar2, obar, rtol=1e-12, atol=1e-12)


def test_zip_guard_fires_when_both_logits_are_zero():
    """KeepKV "numerical stability": the key denominator vanishes when both logits are 0;
    then k_r = (k_e + k_c)/2."""
    d = 8
    ke, kc = RNG.standard_normal(d), RNG.standard_normal(d)
    k_r, v_r, p_r, guarded = zip_merge(ke, np.ones(d), 2, 0.0, kc, np.zeros(d), 1, 0.0)
    assert guarded
    np.testing.assert_allclose(k_r, 0.5 * (ke + kc), rtol=1e-15)
    np.testing.assert_allclose(v_r, np.full(d, 2 / 3), rtol=1e-15)   # weights p_e : p_c = 2 : 1
    assert p_r == 3


def test_cosine_partner_brute_force_and_ties():
    K = np.array([[1.0, 0.0], [2.0, 0.0], [0.0, 1.0], [3.0, 0.0], [1.0, 1.0]])
    pos = np.array([10, 4, 7, 2, 1])
    # rows 1 and 3 are both at cosine 1 with row 0: the lower position (row 3, pos 2) wins
    assert cosine_partner(K, 0, pos) == 3
    # brute force on random keys
    for _ in range(20):
        K = RNG.standard_normal((9, 5))
        pos = RNG.permutation(50)[:9]
        e = int(RNG.integers(0, 9))
        cos = [(K[e] @ K[j]) / np.linalg.norm(K[e]) / np.linalg.norm(K[j]) for j in range(9)]
        cand = [j for j in range(9) if j != e]
        assert cosine_partner(K, e, pos) == max(cand, key=lambda j: (cos[j], -pos[j]))


def test_compact_keeps_survivors_in_slot_order():
    arrays = {"K": np.arange(2 * 6 * 3).reshape(2, 6, 3), "pos": np.array([5, 1, 9, 3, 0, 8])}
    out = compact(arrays, [1, 4], {"K": 1})
    np.testing.assert_array_equal(out["pos"], [5, 9, 3, 8])
    np.testing.assert_array_equal(out["K"], arrays["K"][:, [0, 2, 3, 5]])

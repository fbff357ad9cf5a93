"""Pins of the oracle's MomentKV moment-informed eviction (CPU only).

The residual r_j and the score alpha_j ||r_j|| are tied to things other than
their own formula:
  * closed forms: no evicted token (r_j = v_j), one evicted token (S_tilde = 0,
    r_j = v_j - v_e);
  * an evicted set whose key scatter is sqrt(d) times the identity makes the
    moment model exact for values that are affine in the keys (zero residual),
    and leaves any extra part of a value as its residual; the wrong scale,
    sign or orientation of S_tilde fails it;
  * the empirical covariance written from the evicted rows (the definition on
    the page) against the running-sum identity the oracle uses;
  * invariance under a common shift of every key or every value, and under
    duplicating the evicted set;
  * the sequential rule: the second eviction is scored with the first folded
    in, checked against the closed form of that round.
"""
import numpy as np

import oracle
from oracle.moment_evict import moment_informed_evict, moment_residuals, moment_scores

RNG = np.random.default_rng(7)
D = 16
TAU = 1.0 / np.sqrt(D)


def _mom_from_rows(KE, VE):
    if len(KE) == 0:
        return {"n": 0, "sk": np.zeros(D), "sv": np.zeros(D), "S": np.zeros((D, D))}
    m = oracle.fold_moments(oracle.empty_moments(1, D), np.asarray(KE)[None], np.asarray(VE)[None])
    return {"n": m["n"], "sk": m["sk"][0], "sv": m["sv"][0], "S": m["S"][0]}


def _alpha(L):
    x = RNG.standard_normal(L)
    e = np.exp(x - x.max())
    return e / e.sum()


def test_no_evicted_tokens_residual_is_the_value():
    K, V = RNG.standard_normal((7, D)), RNG.standard_normal((7, D))
    r = moment_residuals(K, V, _mom_from_rows([], []), TAU)
    assert np.array_equal(r, V)
    a = _alpha(7)
    np.testing.assert_allclose(moment_scores(K, V, a, _mom_from_rows([], []), TAU),
                               a * np.linalg.norm(V, axis=1), rtol=1e-14)


def test_one_evicted_token_residual_is_the_value_difference():
    """n_e = 1: k_bar = k_e, v_bar = v_e and S_tilde = v_e k_e^T - v_e k_e^T = 0."""
    ke, ve = RNG.standard_normal(D), RNG.standard_normal(D)
    K, V = RNG.standard_normal((9, D)), RNG.standard_normal((9, D))
    r = moment_residuals(K, V, _mom_from_rows([ke], [ve]), TAU)
    np.testing.assert_allclose(r, V - ve[None], rtol=0, atol=1e-14)


def _exact_evicted_set(scatter_factor=1.0, rotate=True):
    """Evicted keys k0 +- sigma u_a over an orthonormal basis u_a: the key scatter
    sum (k - k_bar)(k - k_bar)^T / n_e is sigma^2 / d times the identity;
    sigma^2 = d / tau makes tau * scatter = identity."""
    Q = np.linalg.qr(RNG.standard_normal((D, D)))[0] if rotate else np.eye(D)
    sigma = np.sqrt(scatter_factor * D / TAU)
    k0 = RNG.standard_normal(D)
    KE = np.vstack([k0 + sigma * Q[:, a] for a in range(D)] + [k0 - sigma * Q[:, a] for a in range(D)])
    return KE


def test_affine_values_have_zero_residual_under_an_isotropic_evicted_set():
    M = RNG.standard_normal((D, D))            # not symmetric: a transposed S_tilde fails
    c0 = RNG.standard_normal(D)
    KE = _exact_evicted_set()
    VE = c0[None] + KE @ M.T
    mom = _mom_from_rows(KE, VE)
    K = 3.0 * RNG.standard_normal((11, D))
    V = c0[None] + K @ M.T
    r = moment_residuals(K, V, mom, TAU)
    assert np.abs(r).max() < 1e-9 * np.abs(V).max()
    # an extra part of each value is its residual
    W = RNG.standard_normal((11, D))
    np.testing.assert_allclose(moment_residuals(K, V + W, mom, TAU), W, rtol=0, atol=1e-9)
    # twice the scatter over-corrects: r = -M (k - k_bar)
    KE2 = _exact_evicted_set(scatter_factor=2.0)
    VE2 = c0[None] + KE2 @ M.T
    kbar2 = KE2.mean(axis=0)
    np.testing.assert_allclose(moment_residuals(K, c0[None] + K @ M.T, _mom_from_rows(KE2, VE2), TAU),
                               -(K - kbar2[None]) @ M.T, rtol=0, atol=1e-8)


def test_running_sum_identity_matches_the_empirical_covariance():
    """S_tilde = sum_E v_i (k_i - k_bar)^T written from the evicted rows (pure Python)."""
    KE, VE = RNG.standard_normal((5, D)), RNG.standard_normal((5, D))
    K, V = RNG.standard_normal((4, D)), RNG.standard_normal((4, D))
    n = len(KE)
    kbar = [sum(KE[i][b] for i in range(n)) / n for b in range(D)]
    vbar = [sum(VE[i][a] for i in range(n)) / n for a in range(D)]
    St = [[sum(VE[i][a] * (KE[i][b] - kbar[b]) for i in range(n)) for b in range(D)] for a in range(D)]
    expect = np.array([[V[j][a] - vbar[a] - TAU * sum(St[a][b] * (K[j][b] - kbar[b]) for b in range(D)) / n
                        for a in range(D)] for j in range(len(K))])
    np.testing.assert_allclose(moment_residuals(K, V, _mom_from_rows(KE, VE), TAU), expect, rtol=0, atol=1e-12)


def test_shift_and_duplication_invariance():
    KE, VE = RNG.standard_normal((6, D)), RNG.standard_normal((6, D))
    K, V = RNG.standard_normal((8, D)), RNG.standard_normal((8, D))
    base = moment_residuals(K, V, _mom_from_rows(KE, VE), TAU)
    ck, cv = 5.0 * RNG.standard_normal(D), 5.0 * RNG.standard_normal(D)
    np.testing.assert_allclose(moment_residuals(K + ck, V, _mom_from_rows(KE + ck, VE), TAU), base, atol=1e-11)
    np.testing.assert_allclose(moment_residuals(K, V + cv, _mom_from_rows(KE, VE + cv), TAU), base, atol=1e-11)
    np.testing.assert_allclose(moment_residuals(K, V, _mom_from_rows(np.vstack([KE, KE]), np.vstack([VE, VE])), TAU),
                               base, atol=1e-12)


def test_sequential_eviction_rescores_after_each_fold():
    """From empty sums: round 1 scores alpha_j ||v_j||; after evicting e1 the sums
    hold one token, so round 2 scores alpha_j ||v_j - v_e1|| / (1 - alpha_e1)."""
    L = 12
    K, V = RNG.standard_normal((L, D)), RNG.standard_normal((L, D))
    a = _alpha(L)
    pos = np.arange(L) + 100
    order, mom, first, rounds = moment_informed_evict(K, V, a, pos, _mom_from_rows([], []), L - 2, TAU)
    e1 = int(np.argmin(a * np.linalg.norm(V, axis=1)))
    assert order[0] == e1
    s2 = a * np.linalg.norm(V - V[e1][None], axis=1) / (1.0 - a[e1])
    s2[e1] = np.inf
    assert order[1] == int(np.argmin(s2))
    np.testing.assert_allclose(rounds[1], s2, rtol=1e-13)
    want = _mom_from_rows(K[order], V[order])
    assert mom["n"] == 2
    for key in ("sk", "sv", "S"):
        np.testing.assert_allclose(mom[key], want[key], rtol=1e-13, atol=1e-13)


def test_zero_weight_tokens_go_first_in_position_order():
    L = 10
    K, V = RNG.standard_normal((L, D)), RNG.standard_normal((L, D))
    a = _alpha(L)
    a[[2, 5, 7]] = 0.0
    pos = np.array([50, 40, 30, 20, 10, 45, 5, 35, 1, 2])
    order, *_ = moment_informed_evict(K, V, a / a.sum(), pos, _mom_from_rows(RNG.standard_normal((3, D)),
                                                                              RNG.standard_normal((3, D))), L - 3, TAU)
    assert list(order) == [2, 7, 5]          # score 0 each: positions 30, 35, 45

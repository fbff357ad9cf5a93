"""Pins of the oracle's KeepKV periodic refresh (CPU only).

Tied to things other than the composition itself:
  * the refresh clears the accumulated error: with rows kept in float64 and no guarded
    merge, attention of the current step's (group-mean) query over the refreshed cache,
    votes included, equals attention over the full reloaded KV -- softmax attention written
    out here in torch float64 -- while an older query of the window is not reproduced;
  * the utilities are eq. (15)'s window sum restarted for every reloaded token: a token that
    no merge touched holds the window sum computed by brute force here, and the live
    utilities add up to 1 - alpha^n_win (every causal softmax row sums to 1 and a merge adds
    the two utilities);
  * votes sum to the number of reloaded tokens; the protected (most recent) tokens keep their
    rows and vote 1; the cache ends at the budget.
"""
import math

import numpy as np
import torch

from oracle.keepkv_refresh import refresh

RNG = np.random.default_rng(23)
D = 16
TAU = 1.0 / math.sqrt(D)


def _full(N, G, n_win):
    K = RNG.standard_normal((N, D))
    V = RNG.standard_normal((N, D))
    q_win = RNG.standard_normal((G, n_win, D))
    return K, V, np.arange(N), q_win


def _attend(q, K, V, votes):
    """Vote-weighted softmax attention in torch float64: o = sum p e^l v / sum p e^l, lse = ln sum p e^l."""
    qt, Kt, Vt = (torch.as_tensor(x, dtype=torch.float64) for x in (q, K, V))
    lg = TAU * (qt @ Kt.T) + torch.log(torch.as_tensor(votes, dtype=torch.float64))
    lse = torch.logsumexp(lg, dim=-1)
    o = torch.softmax(lg, dim=-1) @ Vt
    return o.numpy(), lse.numpy()


def _live(res):
    lv = res["live"]
    return res["K"][lv], res["V"][lv], res["votes"][lv]


def test_refresh_is_lossless_for_the_current_query():
    N, B, n_win = 40, 12, 6
    K, V, pos, q_win = _full(N, 1, n_win)
    q_ref = q_win[:, -1, :]                                     # the current step's query
    res = refresh(K, V, pos, q_win, q_ref, TAU, 0.8, B, protect_from=N - 3)
    assert not res["guarded"] and res["live"].sum() == B
    Kc, Vc, pc = _live(res)
    o_full, lse_full = _attend(q_ref, K, V, np.ones(N))
    o_c, lse_c = _attend(q_ref, Kc, Vc, pc)
    np.testing.assert_allclose(o_c, o_full, rtol=0, atol=1e-10)
    np.testing.assert_allclose(lse_c, lse_full, rtol=0, atol=1e-10)
    # an older window query is not reproduced: the merges used the current query's scores
    q_old = q_win[:, 0, :]
    assert np.abs(_attend(q_old, Kc, Vc, pc)[0] - _attend(q_old, K, V, np.ones(N))[0]).max() > 1e-6


def test_refresh_is_lossless_for_the_group_mean_query():
    N, B, G, n_win = 36, 10, 4, 5
    K, V, pos, q_win = _full(N, G, n_win)
    q_ref = q_win[:, -1, :]
    res = refresh(K, V, pos, q_win, q_ref, TAU, 0.9, B, protect_from=N)
    assert not res["guarded"]
    Kc, Vc, pc = _live(res)
    qbar = q_ref.mean(axis=0, keepdims=True)
    np.testing.assert_allclose(_attend(qbar, Kc, Vc, pc)[0], _attend(qbar, K, V, np.ones(N))[0], rtol=0, atol=1e-10)


def _window_sum_brute(K, q_win, alpha, i):
    """S_i = sum_j (1 - alpha) alpha^(n_win-1-j) * mean_g softmax_j(i), causal by index, in loops."""
    G, n_win, _ = q_win.shape
    N = K.shape[0]
    total = 0.0
    for j in range(n_win):
        last = N - n_win + j
        if i > last:
            continue
        acc = 0.0
        for g in range(G):
            lg = [TAU * float(np.dot(q_win[g, j], K[k])) for k in range(last + 1)]
            mx = max(lg)
            z = sum(math.exp(x - mx) for x in lg)
            acc += math.exp(lg[i] - mx) / z
        total += (1 - alpha) * alpha ** (n_win - 1 - j) * acc / G
    return total


def test_refresh_restarts_the_ema_window_sum():
    N, B, G, n_win, alpha = 30, 9, 2, 4, 0.7
    K, V, pos, q_win = _full(N, G, n_win)
    res = refresh(K, V, pos, q_win, q_win[:, -1, :], TAU, alpha, B, protect_from=N - 2)
    touched = set()
    for s_, g_ in res["pairs"]:
        touched.update((s_, g_))
    untouched = [i for i in range(N) if i not in touched]
    assert untouched
    for i in untouched:
        assert abs(res["m"][i] - _window_sum_brute(K, q_win, alpha, i)) <= 1e-12
    np.testing.assert_allclose(res["m"][res["live"]].sum(), 1 - alpha ** n_win, rtol=1e-12)


def test_refresh_votes_budget_and_protected_tokens():
    N, B, n_win, R = 50, 14, 8, 5
    K, V, pos, q_win = _full(N, 4, n_win)
    res = refresh(K, V, pos, q_win, q_win[:, -1, :], TAU, 0.85, B, protect_from=N - R)
    lv = res["live"]
    assert lv.sum() == B
    assert res["votes"][lv].sum() == N
    for i in range(N - R, N):
        assert lv[i] and res["votes"][i] == 1
        np.testing.assert_array_equal(res["K"][i], K[i])
        np.testing.assert_array_equal(res["V"][i], V[i])

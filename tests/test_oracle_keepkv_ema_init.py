"""Pins of the oracle's KeepKV EMA window initialisation and bias correction (CPU only).

Tied to things other than the window sum itself:
  * the EMA recursion m <- alpha m + (1 - alpha) s run from zero over the window, each s
    taken from a decode step over a cache that grows by one prompt token per step (the
    oracle's attend_unit, pinned to torch elsewhere, and update_utility, pinned to its
    closed form);
  * one window query: (1 - alpha) times the group mean of torch's softmax;
  * the utilities sum to 1 - alpha^n_win (every step's weights sum to 1);
  * causality: the last key is seen by the last query only;
  * bias correction: the corrected EMA of a constant score from a zero state is that
    constant at every step, and the host helper gives the same factor.
"""
import math

import numpy as np
import torch

from oracle import attend_unit, update_utility
from oracle.keepkv_ema_init import ema_window_init, predicted_scores

RNG = np.random.default_rng(23)
D = 16
TAU = 1.0 / math.sqrt(D)


def test_equals_the_recursion_over_a_growing_cache():
    G, N, n_win, alpha = 4, 40, 9, 0.8
    K = RNG.standard_normal((N, D)) * 2.0
    q_win = RNG.standard_normal((G, n_win, D))
    m = np.zeros(N)
    for j in range(n_win):
        L = N - n_win + j + 1                      # the cache after appending the row's own token
        _, a, _, _ = attend_unit(q_win[:, j, :], K[:L], np.zeros((L, D)), None, TAU)
        s = np.zeros(N)
        s[:L] = a.mean(axis=0)
        m = update_utility(m, s, "ema", alpha)
    np.testing.assert_allclose(ema_window_init(q_win, K, TAU, alpha), m, rtol=1e-12, atol=1e-15)


def test_one_query_is_the_scaled_softmax():
    G, N, alpha = 2, 30, 0.9
    K = RNG.standard_normal((N, D))
    q = RNG.standard_normal((G, 1, D))
    ref = torch.softmax(torch.tensor(q[:, 0, :] @ K.T * TAU, dtype=torch.float64), dim=-1).mean(dim=0).numpy()
    np.testing.assert_allclose(ema_window_init(q, K, TAU, alpha), (1 - alpha) * ref, rtol=1e-12)


def test_sum_and_causality():
    G, N, n_win, alpha = 4, 50, 12, 0.7
    K = RNG.standard_normal((N, D))
    q = RNG.standard_normal((G, n_win, D))
    m = ema_window_init(q, K, TAU, alpha)
    np.testing.assert_allclose(m.sum(), 1 - alpha ** n_win, rtol=1e-12)
    # the last key is seen only by the last window row
    _, a, _, _ = attend_unit(q[:, -1, :], K, np.zeros((N, D)), None, TAU)
    np.testing.assert_allclose(m[-1], (1 - alpha) * a.mean(axis=0)[-1], rtol=1e-12)
    assert np.all(m > 0)


def test_bias_correction_recovers_a_constant_score():
    alpha = 0.9
    s = RNG.random(7)
    S = np.zeros(7)
    for t in range(1, 25):
        S = update_utility(S, s, "ema", alpha)
        np.testing.assert_allclose(predicted_scores(S, alpha, t), s, rtol=1e-12)

"""Pins of the oracle's utility rules and bottom-k selection (CPU only).

InertiaKV §3.1 eqs. (2)-(4); KeepKV eq. (15); MomentKV Algorithm 1 phase 1.
"""
import itertools

import numpy as np
import pytest

from oracle import bottom_k, bottom_k_one_at_a_time, top_k_keep, update_utility

RNG = np.random.default_rng(99)


def test_ema_closed_form():
    """m_T = alpha^T m_0 + (1 - alpha) sum_t alpha^(T - t) s_t."""
    L, T, alpha = 17, 40, 0.9
    m0 = RNG.random(L)
    S = RNG.random((T, L))
    m = m0
    for t in range(T):
        m = update_utility(m, S[t], "ema", alpha)
    closed = alpha ** T * m0 + (1 - alpha) * sum(alpha ** (T - 1 - t) * S[t] for t in range(T))
    np.testing.assert_allclose(m, closed, rtol=1e-13)


def test_keepkv_window_initialisation_matches_recursion():
    """KeepKV eq. (15): S^L = sum_{k=L-w}^{L} (1-alpha) alpha^{L-k} s^k equals the
    recursion run from zero over the window's w + 1 scores."""
    w, alpha = 32, 0.8
    s = RNG.random((w + 1, 9))
    S = np.zeros(9)
    for k in range(w + 1):
        S = update_utility(S, s[k], "ema", alpha)
    closed = sum((1 - alpha) * alpha ** (w - k) * s[k] for k in range(w + 1))
    np.testing.assert_allclose(S, closed, rtol=1e-13)


def test_cumulative_and_single():
    s = RNG.random((5, 6))
    m = np.zeros(6)
    for t in range(5):
        m = update_utility(m, s[t], "cumulative")
    np.testing.assert_allclose(m, s.sum(axis=0), rtol=1e-15)
    np.testing.assert_array_equal(update_utility(m, s[3], "single"), s[3])


def test_layer_then_step_chain():
    """InertiaKV §3.1: the EMA state is updated after every compressed layer, so over
    T steps of Lyr layers the weight of score (t, l) is (1-alpha) alpha^(T*Lyr - 1 - (t*Lyr + l))."""
    T, Lyr, alpha = 3, 5, 0.8
    s = RNG.random((T, Lyr, 4))
    m = np.zeros(4)
    for t in range(T):
        for l in range(Lyr):
            m = update_utility(m, s[t, l], "ema", alpha)
    n = T * Lyr
    closed = sum((1 - alpha) * alpha ** (n - 1 - (t * Lyr + l)) * s[t, l]
                 for t in range(T) for l in range(Lyr))
    np.testing.assert_allclose(m, closed, rtol=1e-13)


def _brute_bottom_k(values, pos, k):
    """Exhaustive: the unique subset E of size k whose every key beats every kept key
    under (value, pos) lexicographic order."""
    n = len(values)
    keys = list(zip(values, pos))
    found = []
    for E in itertools.combinations(range(n), k):
        R = [i for i in range(n) if i not in E]
        if not E or not R or max(keys[i] for i in E) < min(keys[i] for i in R):
            found.append(E)
    assert len(found) == 1
    return np.array(sorted(found[0]), dtype=np.int64)


@pytest.mark.parametrize("trial", range(30))
def test_bottom_k_matches_exhaustive_enumeration(trial):
    n = int(RNG.integers(1, 11))
    pool = np.array([0.0, 0.5, 1.0, 5e-324, 2.2e-308, 0.25])    # heavy ties and subnormals
    values = RNG.choice(pool, size=n)
    pos = RNG.permutation(1000)[:n]
    for k in range(0, n + 1):
        E = bottom_k(values, pos, k)
        np.testing.assert_array_equal(E, _brute_bottom_k(list(values), list(pos), k))
        np.testing.assert_array_equal(E, bottom_k_one_at_a_time(values, pos, k))


def test_negative_zero_ties_with_zero():
    values = np.array([0.0, -0.0, 0.0])
    pos = np.array([5, 9, 2])
    np.testing.assert_array_equal(bottom_k(values, pos, 1), [2])
    np.testing.assert_array_equal(bottom_k(values, pos, 2), [0, 2])


def test_top_k_keep_brute_force():
    for trial in range(20):
        n = int(RNG.integers(1, 10))
        s = RNG.choice(np.array([0.1, 0.2, 0.3, 0.0]), size=n)
        K = int(RNG.integers(0, n + 1))
        keep = top_k_keep(s, K)
        # exhaustive: kept set = unique K-subset whose keys all beat the rest under (s, index)
        keys = [(s[i], i) for i in range(n)]
        found = [set(c) for c in itertools.combinations(range(n), K)
                 if not c or len(c) == n or min(keys[i] for i in c) > max(keys[j] for j in range(n) if j not in c)]
        assert len(found) == 1
        assert set(np.flatnonzero(keep)) == found[0]

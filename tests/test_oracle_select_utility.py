"""Pins of the oracle's utility rules and bottom-k selection (CPU only).

InertiaKV §3.1 eqs. (2)-(4); KeepKV eq. (15); MomentKV Algorithm 1 phase 1.
"""
import itertools

import numpy as np
import pytest

from oracle import bottom_k, bottom_k_one_at_a_time, bottom_k_protected, keep_jaccard, top_k_keep, update_utility

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


@pytest.mark.parametrize("trial", range(20))
def test_protected_selection_matches_exhaustive_enumeration(trial):
    """InertiaKV's third lazy alternative: entries at positions >= protect_from rank after all
    others. Exhaustive: the unique k-subset whose keys (protected, value, pos) all beat the rest."""
    n = int(RNG.integers(1, 10))
    values = RNG.choice([0.0, 0.5, 1.0], size=n)
    pos = RNG.permutation(n) + 3
    k = int(RNG.integers(0, n + 1))
    bound = int(RNG.integers(3, n + 4))
    keys = [(int(pos[i] >= bound), values[i], pos[i]) for i in range(n)]
    found = []
    for E in itertools.combinations(range(n), k):
        R = [i for i in range(n) if i not in E]
        if not E or not R or max(keys[i] for i in E) < min(keys[i] for i in R):
            found.append(E)
    assert len(found) == 1
    assert np.array_equal(bottom_k_protected(values, pos, k, bound), np.array(sorted(found[0]), dtype=np.int64))


def test_protected_selection_special_cases():
    values = RNG.random(30)
    pos = RNG.permutation(30)
    # nothing protected, or everything protected: the plain selection
    assert np.array_equal(bottom_k_protected(values, pos, 7, 10 ** 6), bottom_k(values, pos, 7))
    assert np.array_equal(bottom_k_protected(values, pos, 7, -1), bottom_k(values, pos, 7))
    # enough unprotected entries: the plain selection among them
    un = np.flatnonzero(pos < 20)
    got = bottom_k_protected(values, pos, 5, 20)
    assert np.array_equal(got, np.sort(un[bottom_k(values[un], pos[un], 5)]))


def test_keep_jaccard():
    """Jaccard of two kept sets: 1 for identical or two empty sets, 0 for disjoint ones, and
    the count ratio written with plain loops otherwise."""
    assert keep_jaccard(np.zeros(5), np.zeros(5)) == 1.0
    a = RNG.random(40) < 0.5
    assert keep_jaccard(a, a) == 1.0
    assert keep_jaccard(a, ~a) == 0.0
    for _ in range(10):
        a, b = RNG.random(60) < 0.4, RNG.random(60) < 0.6
        both = sum(1 for i in range(60) if a[i] and b[i])
        either = sum(1 for i in range(60) if a[i] or b[i])
        assert keep_jaccard(a, b) == both / either

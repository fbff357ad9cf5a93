"""Pins of the oracle's vote-weighted attention (CPU only).

KeepKV notes eq. (1), (6), (22)-(23); eqs. (2)-(3); MomentKV §2 eq. (3).
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import attend_unit, scope_score

RNG = np.random.default_rng(1234)


def _rand(G=4, L=37, d=16, scale_k=1.0):
    q = RNG.standard_normal((G, d))
    K = RNG.standard_normal((L, d)) * scale_k
    V = RNG.standard_normal((L, d))
    return q, K, V


def _sdpa(q, K, V, scale):
    """Textbook softmax attention from torch's own float64 kernel."""
    qt = torch.from_numpy(q)[None, :, None, :]                  # [1, G, 1, d]
    Kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1)
    Vt = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, Kt, Vt, scale=scale)
    return o[0, :, 0].numpy()


@pytest.mark.parametrize("L", [1, 2, 37, 300])
def test_all_ones_votes_is_textbook_attention(L):
    q, K, V = _rand(L=L, d=32, scale_k=2.0)
    tau = 1 / np.sqrt(32)
    for votes in (None, np.ones(L, dtype=np.int64)):
        logits, a, o, lse = attend_unit(q, K, V, votes, tau)
        np.testing.assert_allclose(o, _sdpa(q, K, V, tau), rtol=1e-12, atol=1e-13)
        ref_lse = torch.logsumexp(torch.from_numpy(tau * q @ K.T), dim=1).numpy()
        np.testing.assert_allclose(lse, ref_lse, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(a.sum(axis=1), 1.0, rtol=1e-13)


def test_constant_vote_changes_nothing_but_lse():
    q, K, V = _rand()
    tau = 0.25
    _, a1, o1, l1 = attend_unit(q, K, V, None, tau)
    _, a7, o7, l7 = attend_unit(q, K, V, np.full(K.shape[0], 7), tau)
    np.testing.assert_allclose(o7, o1, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a7, a1, rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(l7, l1 + np.log(7.0), rtol=1e-14)


def test_integer_votes_equal_duplicated_tokens():
    """KeepKV notes: an entry with p votes acts as p identical copies."""
    q, K, V = _rand(L=11)
    tau = 0.3
    votes = np.array([1, 3, 1, 2, 5, 1, 1, 4, 2, 1, 3])
    _, a, o, lse = attend_unit(q, K, V, votes, tau)
    idx = np.repeat(np.arange(len(votes)), votes)
    _, a_dup, o_dup, lse_dup = attend_unit(q, K[idx], V[idx], None, tau)
    np.testing.assert_allclose(o, o_dup, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_dup, rtol=1e-13)
    summed = np.zeros_like(a)
    np.add.at(summed.T, idx, a_dup.T)
    np.testing.assert_allclose(a, summed, rtol=1e-12, atol=1e-16)


def test_zero_vote_equals_removal():
    q, K, V = _rand(L=9)
    votes = np.array([1, 0, 2, 1, 0, 1, 1, 3, 1])
    _, a, o, lse = attend_unit(q, K, V, votes, 0.5)
    keep = votes > 0
    _, a_r, o_r, lse_r = attend_unit(q, K[keep], V[keep], votes[keep], 0.5)
    np.testing.assert_allclose(o, o_r, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, lse_r, rtol=1e-13)
    assert np.all(a[:, ~keep] == 0)


def test_eviction_identity():
    """KeepKV notes eq. (3): o' over R minus {e} = (o - A_e v_e) / (1 - A_e), with votes."""
    q, K, V = _rand(G=2, L=13)
    votes = RNG.integers(1, 4, size=13)
    _, a, o, _ = attend_unit(q, K, V, votes, 0.4)
    for e in range(13):
        keep = np.arange(13) != e
        _, _, o_e, _ = attend_unit(q, K[keep], V[keep], votes[keep], 0.4)
        A_e = a[:, e:e + 1]
        np.testing.assert_allclose(o_e, (o - A_e * V[e]) / (1 - A_e), rtol=1e-11, atol=1e-13)


def test_lossless_eviction_when_weight_is_zero():
    """KeepKV notes: the perturbation vanishes iff A_e = 0. Build A_e = 0 two ways:
    a key far opposite the (single) query so exp underflows in float64, and a zero vote."""
    q, K, V = _rand(G=1, L=10)
    K[4] = -1e4 * q[0] / np.linalg.norm(q[0])
    votes = np.ones(10, dtype=np.int64)
    votes[7] = 0
    _, a, o, _ = attend_unit(q, K, V, votes, 1.0)
    assert a[0, 4] == 0.0 and a[0, 7] == 0.0
    for e in (4, 7):
        keep = np.arange(10) != e
        _, _, o_e, _ = attend_unit(q, K[keep], V[keep], votes[keep], 1.0)
        np.testing.assert_allclose(o_e, o, rtol=1e-15, atol=1e-15)


def test_retained_evicted_split():
    """MomentKV §2, eq. (3): f = w_R f_R + w_E f_E with w_R = Z_R / Z, from lse."""
    q, K, V = _rand(G=3, L=40)
    _, _, f, lse = attend_unit(q, K, V, None, 0.35)
    for trial in range(5):
        E = RNG.random(40) < 0.3
        _, _, fR, lR = attend_unit(q, K[~E], V[~E], None, 0.35)
        _, _, fE, lE = attend_unit(q, K[E], V[E], None, 0.35)
        wR = np.exp(lR - lse)[:, None]
        wE = np.exp(lE - lse)[:, None]
        np.testing.assert_allclose(wR + wE, 1.0, rtol=1e-13)
        np.testing.assert_allclose(wR * fR + wE * fE, f, rtol=1e-12, atol=1e-13)


def test_empty_and_all_zero_votes():
    q, K, V = _rand(G=2, L=0)
    _, a, o, lse = attend_unit(q, K, V, None, 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    q, K, V = _rand(G=2, L=3)
    _, a, o, lse = attend_unit(q, K, V, np.zeros(3), 1.0)
    assert np.all(o == 0) and np.all(a == 0) and np.all(np.isneginf(lse))


def test_scope_score_is_head_mean():
    """InertiaKV §3.1 eq. (1): s(i) = (1/H) sum_h a^(h)(i); it is a distribution."""
    q, K, V = _rand(G=4, L=25)
    _, a, _, _ = attend_unit(q, K, V, None, 0.3)
    s = scope_score([a[:2], a[2:]])
    np.testing.assert_allclose(s, a.mean(axis=0), rtol=1e-15)
    np.testing.assert_allclose(s.sum(), 1.0, rtol=1e-14)
    # One head: the score is that head's last-query weight.
    np.testing.assert_array_equal(scope_score([a[1:2]]), a[1])

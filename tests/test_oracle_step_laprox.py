"""Pins of the oracle's whole decode step and LaProx scoring (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import (ScopeState, StepParams, attend_unit, bottom_k, decode_step, empty_moments,
                    fold_moments, laprox_keep, laprox_scores, update_utility,
                    value_output_norms, window_column_norms)

RNG = np.random.default_rng(2024)


def _state(U, L, d, moments=True):
    return ScopeState(K=RNG.standard_normal((U, L, d)), V=RNG.standard_normal((U, L, d)),
                      votes=np.ones(L, dtype=np.int64), pos=np.arange(L, dtype=np.int64),
                      m=RNG.random(L) * 0.01, moments=empty_moments(U, d) if moments else None)


def test_step_order_append_attend_score_select_fold_compact():
    U, G, L, d, B = 2, 3, 30, 8, 12
    st = _state(U, L, d)
    q = RNG.standard_normal((U, G, d))
    nk, nv = RNG.standard_normal((U, d)), RNG.standard_normal((U, d))
    prm = StepParams(scale=0.3, rule="ema", alpha=0.9, budget=B)
    post, res = decode_step(st, nk, nv, 100, q, prm)
    # output is the pre-eviction attention over the L + 1 entries
    K1 = np.concatenate([st.K, nk[:, None]], axis=1)
    V1 = np.concatenate([st.V, nv[:, None]], axis=1)
    a_all = []
    for u in range(U):
        _, a, o, lse = attend_unit(q[u], K1[u], V1[u], None, 0.3)
        np.testing.assert_allclose(res.o[u], o, rtol=1e-13)
        np.testing.assert_allclose(res.lse[u], lse, rtol=1e-13)
        a_all.append(a)
    s = np.concatenate(a_all).mean(axis=0)
    m = update_utility(np.append(st.m, 0.0), s, "ema", 0.9)
    E = bottom_k(m, np.append(st.pos, 100), L + 1 - B)
    np.testing.assert_array_equal(res.evicted_pos[0], np.sort(np.append(st.pos, 100)[E]))
    assert post.length == B
    # every survivor keeps its row, vote and updated utility
    alive = np.setdiff1d(np.arange(L + 1), E)
    np.testing.assert_array_equal(post.pos, np.append(st.pos, 100)[alive])
    np.testing.assert_array_equal(post.K, K1[:, alive])
    np.testing.assert_allclose(post.m, m[alive], rtol=1e-15)
    ref = fold_moments(empty_moments(U, d), K1[:, E], V1[:, E])
    assert post.moments["n"] == len(E)
    np.testing.assert_allclose(post.moments["S"], ref["S"], rtol=1e-14)


def test_no_eviction_under_budget_and_steady_single_eviction():
    st = _state(1, 5, 4)
    q = RNG.standard_normal((1, 1, 4))
    post, res = decode_step(st, RNG.standard_normal((1, 4)), RNG.standard_normal((1, 4)), 5, q,
                            StepParams(scale=0.5, budget=10))
    assert post.length == 6 and res.evicted_pos[0].size == 0
    post2, res2 = decode_step(post, RNG.standard_normal((1, 4)), RNG.standard_normal((1, 4)), 6, q,
                              StepParams(scale=0.5, budget=6))
    assert post2.length == 6 and res2.evicted_pos[0].size == 1


def test_groups_run_in_order_with_ema_after_each():
    """A scope of 3 groups (layers): the utility sees three EMA updates per step and the
    evictions of an earlier group are gone before a later group attends."""
    U, G, L, d = 3, 2, 10, 4
    st = _state(U, L, d, moments=False)
    q = RNG.standard_normal((U, G, d))
    prm = StepParams(scale=0.5, rule="ema", alpha=0.8, budget=L, groups=3)
    post, res = decode_step(st, RNG.standard_normal((U, d)), RNG.standard_normal((U, d)), 50, q, prm)
    assert res.evicted_pos[0].size == 1 and res.evicted_pos[1].size == 0
    assert res.s_pos[1].size == L
    m = np.append(st.m, 0.0)
    m = update_utility(m, res.s[0], "ema", 0.8)
    keep = ~np.isin(res.s_pos[0], res.evicted_pos[0])
    m = m[keep]
    m = update_utility(m, res.s[1], "ema", 0.8)
    m = update_utility(m, res.s[2], "ema", 0.8)
    np.testing.assert_allclose(post.m, m, rtol=1e-14)


def test_lazy_step_keeps_stale_utility():
    st = _state(1, 8, 4, moments=False)
    q = RNG.standard_normal((1, 2, 4))
    post, res = decode_step(st, RNG.standard_normal((1, 4)), RNG.standard_normal((1, 4)), 8, q,
                            StepParams(scale=0.5, budget=8, score=False))
    assert res.s[0] is None
    # the appended token has utility 0, the stale minimum, so it is the one evicted
    np.testing.assert_array_equal(res.evicted_pos[0], [8])
    np.testing.assert_array_equal(post.m, st.m)


def test_merge_step_is_lossless_for_single_head():
    """KeepKV Theorem 3 through the whole step: with G = 1 the next attention with the same
    query over the merged cache reproduces the step's output."""
    L, d = 16, 8
    st = _state(1, L, d, moments=False)
    st.votes = RNG.integers(1, 4, size=L)
    q = RNG.standard_normal((1, 1, d))
    post, res = decode_step(st, RNG.standard_normal((1, d)), RNG.standard_normal((1, d)), L, q,
                            StepParams(scale=0.35, rule="single", budget=L, merge=True))
    pe, pc, guarded = res.merges[0]
    assert not guarded and post.length == L
    _, _, o2, lse2 = attend_unit(q[0], post.K[0], post.V[0], post.votes, 0.35)
    np.testing.assert_allclose(o2, res.o[0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse2, res.lse[0], rtol=1e-12)
    assert post.votes.sum() == st.votes.sum() + 1


# ---------------------------------------------------------------- LaProx

def _lap_inputs(n_layers=2, H=4, n_kv=2, N=40, w=5, d=8, D=12):
    Qw = RNG.standard_normal((n_layers, H, w, d))
    K = RNG.standard_normal((n_layers, n_kv, N, d))
    V = RNG.standard_normal((n_layers, n_kv, N, d))
    Wo = 0.1 * RNG.standard_normal((n_layers, H, d, D))
    return Qw, K, V, Wo


def test_laprox_layer_scores_sum_to_one():
    """LaProx key design 2: per-layer normalisation."""
    s = laprox_scores(*_lap_inputs(), scale=0.3)
    np.testing.assert_allclose(s.reshape(s.shape[0], -1).sum(axis=1), 1.0, rtol=1e-13)
    assert np.all(s >= 0)


def test_laprox_single_query_column_norm_is_the_weight():
    """w = 1, G = 1: ||A[:, i]|| is the last query's softmax weight (torch softmax)."""
    d, N = 8, 30
    q = RNG.standard_normal((1, 1, d))
    K = RNG.standard_normal((N, d))
    c = window_column_norms(q, K, 0.4)
    ref = torch.softmax(torch.from_numpy(0.4 * K @ q[0, 0]), dim=0).numpy()
    np.testing.assert_allclose(c, ref, rtol=1e-13)


def test_laprox_causal_window():
    """Row j at position N - w + j sees keys up to that position only: the last w-1 keys
    get weight from fewer rows; key N-1 only from the last row."""
    d, N, w = 4, 12, 3
    Qw = RNG.standard_normal((1, w, d))
    K = RNG.standard_normal((N, d))
    c = window_column_norms(Qw, K, 0.5)
    A_last = torch.softmax(torch.from_numpy(0.5 * K @ Qw[0, -1]), dim=0).numpy()
    np.testing.assert_allclose(c[-1], A_last[-1], rtol=1e-13)
    # a key past every window row cannot exist; a key before the window is seen by all rows
    rows = [torch.softmax(torch.from_numpy(0.5 * K[:N - w + j + 1] @ Qw[0, j]), dim=0).numpy()
            for j in range(w)]
    np.testing.assert_allclose(c[0], np.sqrt(sum(r[0] ** 2 for r in rows)), rtol=1e-13)


def test_laprox_identity_projection_reduces_to_value_norm():
    """With D = d and W_bar = I (each of the G blocks I / G), ||v W_bar|| = ||v||: the
    'attention x ||V||' variant of the LaProx ablation."""
    G, d, N = 4, 6, 25
    Wo = np.stack([np.eye(d) / G] * G)
    V = RNG.standard_normal((N, d))
    np.testing.assert_allclose(value_output_norms(V, Wo), np.linalg.norm(V, axis=1), rtol=1e-13)


def test_laprox_gram_identity():
    """r_i^2 = v_i (W_bar W_bar^T) v_i^T."""
    G, d, D, N = 4, 8, 33, 20
    Wo = RNG.standard_normal((G, d, D))
    V = RNG.standard_normal((N, d))
    Wb = Wo.sum(axis=0)
    gram = np.einsum("na,ab,nb->n", V, Wb @ Wb.T, V)
    np.testing.assert_allclose(value_output_norms(V, Wo) ** 2, gram, rtol=1e-12)


def test_laprox_equal_value_norms_rank_by_attention():
    Qw, K, V, Wo = _lap_inputs(n_layers=1, H=2, n_kv=1, N=20, d=6, D=6)
    Wo[:] = np.eye(6) / 2
    V = V / np.linalg.norm(V, axis=-1, keepdims=True)
    s, parts = laprox_scores(Qw, K, V, Wo, 0.4, return_parts=True)
    np.testing.assert_allclose(parts["r"], 1.0, rtol=1e-13)
    np.testing.assert_allclose(s[0, 0], parts["c"][0, 0] / parts["c"][0, 0].sum(), rtol=1e-13)


def test_laprox_top_k_is_global():
    s = laprox_scores(*_lap_inputs(n_layers=3), scale=0.3)
    keep = laprox_keep(s, 17)
    assert keep.sum() == 17
    assert s[keep].min() >= s[~keep].max()

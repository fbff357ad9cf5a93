"""Pins of the oracle's MomentKV normalisation-corrected output (CPU only).

The corrected output is tied to things other than its own formula: full
attention over R and E (textbook softmax attention of attend_unit) whenever
the first-order estimate is exact (one evicted token; identical evicted keys),
second-order convergence of the error as the evicted keys spread, the Jensen
bias of the mixing weight, and the degenerate cases of Algorithm 1 phase 2.
"""
import numpy as np
import pytest

import oracle

RNG = np.random.default_rng(2024)
D = 16
TAU = 1.0 / np.sqrt(D)


def _split(G=3, nR=9, nE=5, spread=1.0, same_key=False):
    q = RNG.standard_normal((G, D))
    KR, VR = RNG.standard_normal((nR, D)), RNG.standard_normal((nR, D))
    k0 = RNG.standard_normal(D)
    KE = k0 + spread * RNG.standard_normal((nE, D)) if not same_key else np.tile(k0, (nE, 1))
    VE = RNG.standard_normal((nE, D))
    return q, KR, VR, KE, VE


def _mom(KE, VE):
    m = oracle.fold_moments(oracle.empty_moments(1, D), KE[None], VE[None])
    return {"n": m["n"], "sk": m["sk"][0], "sv": m["sv"][0], "S": m["S"][0]}


def _corrected(q, KR, VR, KE, VE):
    _, _, fR, lseR = oracle.attend_unit(q, KR, VR, None, TAU)
    return oracle.corrected_output(fR, lseR, q, _mom(KE, VE), TAU)


def _full(q, KR, VR, KE, VE):
    return oracle.attend_unit(q, np.vstack([KR, KE]), np.vstack([VR, VE]), None, TAU)[2]


def test_no_eviction_returns_the_retained_output():
    q, KR, VR, _, _ = _split()
    _, _, fR, lseR = oracle.attend_unit(q, KR, VR, None, TAU)
    out = oracle.corrected_output(fR, lseR, q, {"n": 0, "sk": np.zeros(D), "sv": np.zeros(D),
                                                 "S": np.zeros((D, D))}, TAU)
    assert np.array_equal(out, fR)


def test_one_evicted_token_is_recovered_exactly():
    """n_e = 1: S_tilde = 0, f_E_hat = v_e and Z_E_hat = e^{tau q.k_e} are exact."""
    for _ in range(5):
        q, KR, VR, KE, VE = _split(nE=1, spread=3.0)
        np.testing.assert_allclose(_corrected(q, KR, VR, KE, VE), _full(q, KR, VR, KE, VE), rtol=0, atol=1e-12)


def test_identical_evicted_keys_are_recovered_exactly():
    """Equal evicted keys: every centred logit is zero, so the estimates are exact."""
    q, KR, VR, KE, VE = _split(nE=6, same_key=True)
    np.testing.assert_allclose(_corrected(q, KR, VR, KE, VE), _full(q, KR, VR, KE, VE), rtol=0, atol=1e-12)


def test_error_is_second_order_in_the_key_spread():
    """Keys k0 + eps u_i: the first-order estimate errs by O(eps^2) (a dropped or
    mis-signed covariance term would leave O(eps))."""
    q = RNG.standard_normal((2, D))
    KR, VR = RNG.standard_normal((7, D)), RNG.standard_normal((7, D))
    k0, U = RNG.standard_normal(D), RNG.standard_normal((8, D))
    VE = RNG.standard_normal((8, D))
    errs = []
    for eps in (0.08, 0.04, 0.02):
        KE = k0 + eps * U
        errs.append(np.abs(_corrected(q, KR, VR, KE, VE) - _full(q, KR, VR, KE, VE)).max())
    for a, b in zip(errs, errs[1:]):
        assert 3.0 < a / b < 5.0, errs
    # the uncorrected retained output is wrong at first order
    KE = k0 + 0.02 * U
    _, _, fR, _ = oracle.attend_unit(q, KR, VR, None, TAU)
    assert np.abs(fR - _full(q, KR, VR, KE, VE)).max() > 100 * errs[-1]


def test_mixing_weight_leans_to_the_retained_set():
    """Z_E_hat <= Z_E (Jensen), so the retained weight is never below the true one."""
    for _ in range(20):
        q, KR, VR, KE, VE = _split(nE=7, spread=2.0)
        _, _, _, lseR = oracle.attend_unit(q, KR, VR, None, TAU)
        _, lnZE = oracle.evicted_estimates(q, _mom(KE, VE), TAU)
        _, _, _, lseE = oracle.attend_unit(q, KE, VE, None, TAU)
        assert np.all(lnZE <= lseE + 1e-12)
        w_hat = 1 / (1 + np.exp(lnZE - lseR))
        w_true = 1 / (1 + np.exp(lseE - lseR))
        assert np.all(w_hat >= w_true - 1e-15)


def test_empty_retained_set_gives_the_evicted_estimate():
    q, _, _, KE, VE = _split(nE=4)
    fE, _ = oracle.evicted_estimates(q, _mom(KE, VE), TAU)
    out = oracle.corrected_output(np.zeros((3, D)), np.full(3, -np.inf), q, _mom(KE, VE), TAU)
    np.testing.assert_array_equal(out, fE)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_extreme_logit_gaps_stay_finite(sign):
    q, KR, VR, KE, VE = _split(nE=3)
    KE = KE + sign * 400.0 * q[0] / np.linalg.norm(q[0]) ** 2 * np.sqrt(D)
    out = _corrected(q, KR, VR, KE, VE)
    assert np.all(np.isfinite(out))

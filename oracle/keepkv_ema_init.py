"""KeepKV's window initialisation of the EMA score state (test infrastructure, fp64).

KeepKV reading notes, "EMA score prediction": eq. (15) sets the state at the end of
prefill (t = L) to the window sum S^L = sum over the last steps k of
(1 - alpha) alpha^(L - k) s^k, the inference algorithm's prefill step 4 applies it, and
eq. (14) predicts the score as S^t / (1 - alpha^t).

Readings (the notes leave these open):
  * s^k is the score of step k's query: the normalised attention weight of each key,
    averaged over the G query heads of the KV head (InertiaKV §3.1 eq. (1) per KV head),
    causal -- step k's query sees the keys at positions <= k, a later key scores 0;
  * the window holds the last n_win prompt queries (the page's w is n_win - 1), row j
    at position N - n_win + j of an N-token prompt.
"""
from __future__ import annotations

import numpy as np

from .attention import attend_unit


def window_scores(q_win, K, scale):
    """s [n_win, N]: s[j, i] = mean over g of softmax_i(scale q_win[g, j] . k_i) over the
    keys i <= N - n_win + j; 0 for the later keys."""
    q_win = np.asarray(q_win, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    G, n_win, d = q_win.shape
    N = K.shape[0]
    s = np.zeros((n_win, N))
    for j in range(n_win):
        last = N - n_win + j
        _, a, _, _ = attend_unit(q_win[:, j, :], K[:last + 1], np.zeros((last + 1, d)), None, scale)
        s[j, :last + 1] = a.mean(axis=0)
    return s


def ema_window_init(q_win, K, scale, alpha):
    """S [N] = sum_j (1 - alpha) alpha^(n_win - 1 - j) s[j] (eq. (15) at the end of prefill)."""
    s = window_scores(q_win, K, scale)
    n_win = s.shape[0]
    weights = (1.0 - alpha) * alpha ** (n_win - 1 - np.arange(n_win, dtype=np.float64))
    return weights @ s


def predicted_scores(S, alpha, t):
    """Eq. (14): s_hat^t = S^t / (1 - alpha^t)."""
    return np.asarray(S, dtype=np.float64) / (1.0 - alpha ** t)

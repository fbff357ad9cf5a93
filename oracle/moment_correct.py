"""MomentKV normalisation-corrected inference (test infrastructure, fp64).

MomentKV summary page, Algorithm 1 phase 2 and §4.2 ("normalisation-corrected
inference"), with the first-order estimate of §4.1: the attention output of
one query head over the retained set R is corrected for the evicted set E,
known only through its running sums (n_e, s_k, s_v, S):

  f_R, Z_R       attention output and partition function over R;
  if n_e = 0:    the output is f_R;
  Z_E_hat      = n_e exp(tau q . k_bar)             (Jensen lower bound of Z_E),
  f_E_hat      = v_bar + tau S_tilde q / n_e        (first-order Taylor estimate),
  w_R          = Z_R / (Z_R + Z_E_hat),
  output       = w_R f_R + (1 - w_R) f_E_hat,

with k_bar = s_k / n_e, v_bar = s_v / n_e, S_tilde = S - s_v s_k^T / n_e and
tau the softmax scale (the page's 1/sqrt(d)). Z_R enters through
lse_R = ln Z_R; the mixing weight is formed from ln Z_E_hat - lse_R (a
logistic of that difference), which is the same ratio without overflow.
"""
from __future__ import annotations

import numpy as np

from .moments import centred_moments


def evicted_estimates(q, mom_unit, scale):
    """(f_E_hat [G, d], ln Z_E_hat [G]) for one unit; mom_unit = {"n", "sk" [d], "sv" [d], "S" [d, d]}
    with n > 0; q [G, d]."""
    q = np.asarray(q, dtype=np.float64)
    n = float(mom_unit["n"])
    kbar, vbar, St = centred_moments({"n": n, "sk": mom_unit["sk"][None], "sv": mom_unit["sv"][None],
                                      "S": mom_unit["S"][None]})
    kbar, vbar, St = kbar[0], vbar[0], St[0]
    fE = vbar[None, :] + scale * (q @ St.T) / n            # (S_tilde q_g)_a = sum_b S_tilde[a][b] q_g[b]
    lnZE = np.log(n) + scale * (q @ kbar)
    return fE, lnZE


def corrected_output(f_R, lse_R, q, mom_unit, scale):
    """Corrected output [G, d] of one unit's G query heads (Algorithm 1, steps 16-21).

    f_R [G, d], lse_R [G] (ln Z_R; -inf for an empty retained set), q [G, d]."""
    f_R = np.asarray(f_R, dtype=np.float64)
    lse_R = np.asarray(lse_R, dtype=np.float64)
    if mom_unit["n"] == 0:
        return f_R.copy()
    fE, lnZE = evicted_estimates(q, mom_unit, scale)
    x = lnZE - lse_R                                        # ln(Z_E_hat / Z_R)
    with np.errstate(over="ignore"):
        w_R = np.where(x > 0, np.exp(-x) / (1.0 + np.exp(-x)), 1.0 / (1.0 + np.exp(x)))
    return w_R[:, None] * f_R + (1.0 - w_R[:, None]) * fE

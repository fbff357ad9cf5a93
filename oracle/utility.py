"""Temporal utility aggregation.

InertiaKV §3.1, eqs. (2)-(4): keep a utility m_t over the live tokens and
update it from the per-step score s_t with one of three rules:
  single      m_t = s_t
  cumulative  m_t = m_{t-1} + s_t
  EMA         m_t = alpha m_{t-1} + (1 - alpha) s_t
The same recursion is KeepKV's eq. (15) for t > L (its score state S^t).
"""
from __future__ import annotations

import numpy as np

SINGLE, CUMULATIVE, EMA = 0, 1, 2
RULES = {"single": SINGLE, "cumulative": CUMULATIVE, "ema": EMA}


def update_utility(m_prev, s, rule, alpha: float = 0.0):
    rule = RULES.get(rule, rule)
    m_prev = np.asarray(m_prev, dtype=np.float64)
    s = np.asarray(s, dtype=np.float64)
    if rule == SINGLE:
        return s.copy()
    if rule == CUMULATIVE:
        return m_prev + s
    if rule == EMA:
        return alpha * m_prev + (1.0 - alpha) * s
    raise ValueError(f"unknown utility rule {rule!r}")

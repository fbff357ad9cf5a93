"""One decode step of a fixed-budget cache scope, in the order the pages give.

Order (MomentKV Algorithm 1 steps 1-2 and phase 1; KeepKV Algorithm, decode
steps 6a-6f; InertiaKV §3.1):
  1. append the new token's key/value rows (vote 1),
  2. attend over every live entry, new one included (the step's output is
     the pre-eviction output),
  3. score: head-averaged weights s(i),
  4. aggregate: utility update m <- rule(m, s),
  5. select the k = L - B lowest-utility entries,
  6. fold the selected rows into the moment statistics (if kept),
  7. remove them (or, in merge mode, ZIP-merge the selected entry into its
     cosine partner and remove it).

A scope is a set of units sharing one slot set. Its units are split into
`groups` consecutive attention groups that run in order, each followed by
its own score/aggregate/select/act (InertiaKV §3.1: the EMA state is updated
after every compressed layer). A per-KV-head scope is one group of one unit.

Readings (the pages leave these open):
  * a new entry's utility starts at 0 before its first update;
  * steps that do not refresh scores (lazy refresh) skip 3-4 and still hold
    the budget with the stale utility; optionally (InertiaKV's third lazy
    alternative) the entries appended since the last refresh are protected
    from selection;
  * merge mode handles one eviction per group step and scopes of one unit.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .attention import attend_unit, scope_score
from .compaction import compact
from .convert import to_f64, round_to_bf16, round_to_f32
from .moments import fold_moments
from .selection import bottom_k, bottom_k_protected
from .utility import update_utility
from .zip_merge import cosine_partner, zip_merge


@dataclass
class ScopeState:
    K: np.ndarray            # [U, L, d] float64
    V: np.ndarray            # [U, L, d] float64
    votes: np.ndarray        # [L] int64
    pos: np.ndarray          # [L] int64
    m: np.ndarray            # [L] float64
    moments: dict | None = None

    @property
    def length(self) -> int:
        return self.K.shape[1]

    def copy(self) -> "ScopeState":
        mom = None if self.moments is None else {k: (v.copy() if isinstance(v, np.ndarray) else v)
                                                 for k, v in self.moments.items()}
        return ScopeState(self.K.copy(), self.V.copy(), self.votes.copy(), self.pos.copy(),
                          self.m.copy(), mom)


@dataclass
class StepParams:
    scale: float
    rule: object = "ema"
    alpha: float = 0.9
    budget: int = 0
    groups: int = 1
    score: bool = True
    merge: bool = False
    eps: float = 1e-6
    row_dtype: str = "f64"   # cache dtype of rows written by a merge: "bf16", "f32" or "f64"
    protect_from: int | None = None   # entries at positions >= this rank after all others in selection


@dataclass
class StepResult:
    o: np.ndarray                       # [U, G, d]
    lse: np.ndarray                     # [U, G]
    s: list = field(default_factory=list)          # per group: s over the live slots, or None
    s_pos: list = field(default_factory=list)      # per group: positions the s entries belong to
    evicted_pos: list = field(default_factory=list)  # per group: sorted evicted positions
    merges: list = field(default_factory=list)     # per group: (pos_e, pos_c, guarded) or None
    m_pre: list = field(default_factory=list)      # per group: utility of every live entry before removal
    m_pos: list = field(default_factory=list)      # per group: positions of those entries


def _round_rows(x, row_dtype):
    if row_dtype == "bf16":
        return to_f64(round_to_bf16(x))
    if row_dtype == "f32":
        return round_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def decode_step(state: ScopeState, new_k, new_v, new_pos, q, prm: StepParams):
    """Returns (post_state, StepResult). Inputs are not modified.

    new_k, new_v: [U, d] or None (no append); new_pos: position of the new token;
    q: [U, G, d] query heads of every unit.
    """
    st = state.copy()
    U = st.K.shape[0]
    q = np.asarray(q, dtype=np.float64)
    G = q.shape[1]
    if new_k is not None:
        st.K = np.concatenate([st.K, np.asarray(new_k, dtype=np.float64)[:, None, :]], axis=1)
        st.V = np.concatenate([st.V, np.asarray(new_v, dtype=np.float64)[:, None, :]], axis=1)
        st.votes = np.append(st.votes, 1)
        st.pos = np.append(st.pos, new_pos)
        st.m = np.append(st.m, 0.0)

    res = StepResult(o=np.zeros((U, G, q.shape[2])), lse=np.zeros((U, G)))
    if U % prm.groups:
        raise ValueError("units must split evenly into groups")
    ug = U // prm.groups
    for g in range(prm.groups):
        units = range(g * ug, (g + 1) * ug)
        a_list, logit_list = [], []
        for u in units:
            logits, a, o, lse = attend_unit(q[u], st.K[u], st.V[u], st.votes, prm.scale)
            res.o[u], res.lse[u] = o, lse
            a_list.append(a)
            logit_list.append(logits)
        if prm.score:
            s = scope_score(a_list)
            st.m = update_utility(st.m, s, prm.rule, prm.alpha)
            res.s.append(s)
            res.s_pos.append(st.pos.copy())
        else:
            res.s.append(None)
            res.s_pos.append(None)

        res.m_pre.append(st.m.copy())
        res.m_pos.append(st.pos.copy())
        k = st.length - prm.budget
        if k <= 0:
            res.evicted_pos.append(np.zeros(0, dtype=np.int64))
            res.merges.append(None)
            continue
        if prm.protect_from is None:
            E = bottom_k(st.m, st.pos, k)
        else:
            E = bottom_k_protected(st.m, st.pos, k, prm.protect_from)
        res.evicted_pos.append(np.sort(st.pos[E]))
        if st.moments is not None:
            st.moments = fold_moments(st.moments, st.K[:, E], st.V[:, E])
        merge_info = None
        if prm.merge:
            if k != 1 or U != 1:
                raise ValueError("merge mode: one eviction per step, one unit per scope")
            e = int(E[0])
            c = cosine_partner(st.K[0], e, st.pos)
            lbar = logit_list[-1].mean(axis=0)            # group-mean logit = logit of mean query
            k_r, v_r, p_r, guarded = zip_merge(st.K[0, e], st.V[0, e], st.votes[e], lbar[e],
                                               st.K[0, c], st.V[0, c], st.votes[c], lbar[c], prm.eps)
            st.K[0, c] = _round_rows(k_r, prm.row_dtype)
            st.V[0, c] = _round_rows(v_r, prm.row_dtype)
            st.votes[c] = p_r
            st.m[c] = st.m[c] + st.m[e]
            merge_info = (int(st.pos[e]), int(st.pos[c]), guarded)
        res.merges.append(merge_info)
        kept = compact({"K": st.K, "V": st.V, "votes": st.votes, "pos": st.pos, "m": st.m}, E,
                       {"K": 1, "V": 1})
        st.K, st.V, st.votes, st.pos, st.m = kept["K"], kept["V"], kept["votes"], kept["pos"], kept["m"]
    return st, res

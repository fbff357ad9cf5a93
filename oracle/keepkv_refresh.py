"""KeepKV's periodic refresh (test infrastructure, fp64).

KeepKV reading notes: the inference algorithm's decode step 6g, the multi-step decode
pipeline of Figure 4 and the paragraph on periodic refresh. The full KV cache is kept in
external (host) memory; every T decode steps it is loaded back and compressed again by ZIP
merging, which clears the error the EMA-predicted merges of the steps in between have
accumulated.

Readings (the notes leave these open):
  * the external store holds every token so far, the prompt's and the decode steps', in
    position order, each with vote 1: the refresh starts from the full KV, not from the
    compressed cache, whose merges are not carried over;
  * "ZIP merging again with the current EMA scores": a reloaded token that had been merged
    away has no EMA state of its own, so the state of every reloaded token is set again by
    eq. (15)'s window form over the last n_win queries (the rule the prefill's step 4
    applies, here over the latest decode steps' queries), and the merges use the exact
    group-mean logits of the current step's query, as the prefill's step 5 uses its last
    query's exact scores: only exact scores make the compressed cache lossless for the
    current query (Theorem 3), which is what clears the accumulated error;
  * protection bound, merged-entry slot and utility, and ties as in prefill merging.

This is the composition of ema_window_init and prefill_merge, both pinned on their own; its
own pins are in tests/test_oracle_keepkv_refresh.py.
"""
from __future__ import annotations

import numpy as np

from .keepkv_ema_init import ema_window_init
from .keepkv_prefill import prefill_merge


def refresh(K_full, V_full, pos, q_win, q_ref, scale, alpha, budget, protect_from, eps=1e-6, row_dtype="f64",
            choose=None):
    """One head's refresh from its full KV.

    K_full, V_full: [N, d] every token so far in position order (pos: [N], increasing);
    q_win: [G, n_win, d] the queries of the last n_win steps (row j at position
    pos[N - n_win + j]); q_ref: [G, d] the current step's query heads. Returns
    prefill_merge's dict over the N reloaded slots (K, V, votes, m, live, pairs, guarded)."""
    K_full = np.asarray(K_full, dtype=np.float64)
    N = K_full.shape[0]
    m = ema_window_init(q_win, K_full, scale, alpha)            # eq. (15), window form
    votes = np.ones(N, dtype=np.int64)
    return prefill_merge(K_full, V_full, votes, pos, m, q_ref, scale, budget, protect_from, eps=eps,
                         row_dtype=row_dtype, choose=choose)

"""LaProx prefill score, per-layer normalisation and model-wide Top-K.

LaProx notes ("Reformulating KV Cache Eviction Problem for Long-Context LLM
Inference"):
  * key design 1: the multi-head output is sum_h A^h (V^h W_O^h); keeping the
    entries that best approximate A x (V W_O) gives the indicator
        p_i  ~  ||A[:, i]||_2 * ||(V W_O)[i, :]||_2 ;
  * key design 2: within a layer the flattened scores of every head are
    normalised to sum to one, s_{l,j} = p_{l,j} / sum_k p_{l,k};
  * key design 3: one Top-K over every (layer, head, token) of the model;
  * training-strategy paragraph: under GQA the attention weights of the
    query heads of one group are averaged; scoring is done once, at the end
    of prefill, from the observation window (the last w queries).

Readings: window row j (0-based) sits at prompt position N - w + j and
attends causally to keys i <= N - w + j; under GQA the projected values of a
KV head use W_bar = sum of the group's W_O^g blocks, since
sum_g Abar (V W_O^g) = Abar (V W_bar).
"""
from __future__ import annotations

import numpy as np

from .selection import top_k_keep


def window_column_norms(Qw, K, scale):
    """c_i = ||Abar[:, i]||_2 for one KV head.

    Qw [G, w, d]: the group's window queries; K [N, d] float64.
    A_{g,j,i} = exp(tau q_{g,j}.k_i) / sum_{i' <= P_j} exp(tau q_{g,j}.k_{i'}) for i <= P_j, else 0;
    Abar = mean over g. Returns c [N].
    """
    Qw = np.asarray(Qw, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    G, w, d = Qw.shape
    N = K.shape[0]
    logits = scale * np.einsum("gjd,nd->gjn", Qw, K)
    P = N - w + np.arange(w)
    causal = np.arange(N)[None, :] <= P[:, None]            # [w, N]
    logits = np.where(causal[None], logits, -np.inf)
    M = logits.max(axis=2, keepdims=True)
    e = np.exp(logits - M)
    A = e / e.sum(axis=2, keepdims=True)
    Abar = A.mean(axis=0)
    return np.sqrt((Abar * Abar).sum(axis=0))


def value_output_norms(V, Wo_group, chunk: int = 4096):
    """r_i = ||v_i W_bar||_2 with W_bar = sum_g W_O^g.

    V [N, d]; Wo_group [G, d, D]. Rows are computed in chunks of tokens only to
    bound memory; each row is the plain product and norm."""
    V = np.asarray(V, dtype=np.float64)
    Wbar = np.asarray(Wo_group, dtype=np.float64).sum(axis=0)
    r = np.empty(V.shape[0])
    for i0 in range(0, V.shape[0], chunk):
        P = V[i0:i0 + chunk] @ Wbar
        r[i0:i0 + chunk] = np.sqrt((P * P).sum(axis=1))
    return r


def laprox_scores(Qw, K, V, Wo, scale, return_parts=False):
    """Normalised scores s [layers, n_kv, N].

    Qw [layers, H, w, d]; K, V [layers, n_kv, N, d]; Wo [layers, H, d, D].
    Query head h belongs to KV head h // G (consecutive grouping)."""
    n_layers, H = Qw.shape[:2]
    n_kv, N = K.shape[1], K.shape[2]
    G = H // n_kv
    c = np.zeros((n_layers, n_kv, N))
    r = np.zeros((n_layers, n_kv, N))
    for l in range(n_layers):
        for h in range(n_kv):
            grp = slice(h * G, (h + 1) * G)
            c[l, h] = window_column_norms(Qw[l, grp], K[l, h], scale)
            r[l, h] = value_output_norms(V[l, h], Wo[l, grp])
    p = c * r
    sigma = p.reshape(n_layers, -1).sum(axis=1)
    s = p / sigma[:, None, None]
    if return_parts:
        return s, {"c": c, "r": r, "p": p, "sigma": sigma}
    return s


def laprox_keep(s, keep_total: int):
    """Keep mask of the model-wide Top-K of the normalised scores (flat index ties)."""
    return top_k_keep(s, keep_total)

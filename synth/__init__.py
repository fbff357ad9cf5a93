"""Seeded synthetic inputs for the fixed-budget decode step and for LaProx scoring.

This module only draws random numbers and casts them to the cache dtype. It
holds none of the method's arithmetic, so both the HIP path (through the
tests and bench.py) and the CPU oracle consume the very same bytes from it.

Every draw comes from a torch generator seeded from a numpy SeedSequence of
(config seed, stream id[, step]); on a GPU device torch uses its counter-based
Philox generator, on the CPU its Mersenne twister. A test always hands the
oracle a host copy of the tensors the GPU consumed, never a regenerated copy.

Streams (ids fixed so that adding a stream never changes another one):
K, V, channel scales, outlier channels, query stream, new keys, new values,
votes, W_O, window queries, initial positions, moment sums, weights.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import LAPROX_WORKLOADS, LaproxWorkload, Workload, WORKLOADS, budget_for  # noqa: F401  (re-export)

S_K, S_V, S_SCALE, S_OUTLIER, S_Q, S_NEWK, S_NEWV, S_VOTES, S_WO, S_QWIN, S_POS, S_MOM, S_ALPHA = range(13)

_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def torch_dtype(name: str) -> torch.dtype:
    return _DTYPES[name]


def _gen(seed: int, stream: int, step: int | None, device) -> torch.Generator:
    words = [int(seed), int(stream)] + ([] if step is None else [int(step)])
    s = int(np.random.SeedSequence(words).generate_state(2, dtype=np.uint32).astype(np.uint64)
            .dot(np.array([1, 1 << 32], dtype=np.uint64)) & np.uint64((1 << 63) - 1))
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(s)
    return g


def _randn(shape, seed, stream, step, device) -> torch.Tensor:
    g = _gen(seed, stream, step, device)
    return torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)


def key_scales(n_units: int, d: int, seed: int, device="cpu", lognormal_sigma=0.5,
               n_outliers=4, outlier_factor=8.0) -> torch.Tensor:
    """Per-(unit, channel) key scale: LogNormal(0, sigma), with `n_outliers`
    distinct channels per unit multiplied by `outlier_factor`. Returns [n_units, d] f32."""
    z = _randn((n_units, d), seed, S_SCALE, None, device)
    c = torch.exp(lognormal_sigma * z)
    if n_outliers > 0:
        g = _gen(seed, S_OUTLIER, None, device)
        r = torch.rand((n_units, d), generator=g, device=device)
        idx = torch.argsort(r, dim=1)[:, :n_outliers]      # n distinct channels per unit
        c.scatter_(1, idx, c.gather(1, idx) * outlier_factor)
    return c


def kv_rows(n_units: int, n_rows: int, d: int, dtype: str, seed: int, device="cpu",
            scales: torch.Tensor | None = None):
    """Initial K, V rows [n_units, n_rows, d] in the cache dtype (cast with
    round-to-nearest-even). K ~ N(0,1) times the unit's channel scales when
    given; V ~ N(0,1). Rows are drawn in blocks of 4096, each block from its
    own stream step, so peak temporary memory stays small."""
    K = torch.empty((n_units, n_rows, d), dtype=_DTYPES[dtype], device=device)
    V = torch.empty_like(K)
    blk = 4096
    for r0 in range(0, n_rows, blk):
        r1 = min(n_rows, r0 + blk)
        step = r0 // blk
        k = _randn((n_units, r1 - r0, d), seed, S_K, step, device)
        if scales is not None:
            k = k * scales[:, None, :].to(device)
        K[:, r0:r1] = k.to(_DTYPES[dtype])
        V[:, r0:r1] = _randn((n_units, r1 - r0, d), seed, S_V, step, device).to(_DTYPES[dtype])
    return K, V


def step_query(step: int, n_units: int, G: int, d: int, dtype: str, seed: int, device="cpu"):
    """Query heads of decode step `step`: [n_units, G, d] ~ N(0,1) in the cache dtype."""
    return _randn((n_units, G, d), seed, S_Q, step, device).to(_DTYPES[dtype])


def step_new_kv(step: int, n_units: int, d: int, dtype: str, seed: int, device="cpu",
                scales: torch.Tensor | None = None):
    """New key/value rows appended at decode step `step`: [n_units, d] each."""
    k = _randn((n_units, d), seed, S_NEWK, step, device)
    if scales is not None:
        k = k * scales.to(device)
    v = _randn((n_units, d), seed, S_NEWV, step, device)
    return k.to(_DTYPES[dtype]), v.to(_DTYPES[dtype])


def prior_votes(n_scopes: int, n_slots: int, seed: int, lam: float = 2.0, device="cpu"):
    """Votes left by earlier merges: 1 + Poisson(lam), int32 [n_scopes, n_slots]."""
    g = _gen(seed, S_VOTES, None, "cpu")
    rate = torch.full((n_scopes, n_slots), float(lam))
    return (1 + torch.poisson(rate, generator=g)).to(torch.int32).to(device)


def initial_positions(n_scopes: int, n_slots: int, context: int, seed: int, device="cpu"):
    """Sorted distinct token positions in [0, context) for a cache that starts
    already compressed to `n_slots` entries: int32 [n_scopes, n_slots]."""
    g = _gen(seed, S_POS, None, "cpu")
    out = torch.empty((n_scopes, n_slots), dtype=torch.int32)
    for s in range(n_scopes):
        out[s] = torch.sort(torch.randperm(context, generator=g)[:n_slots]).values.to(torch.int32)
    return out.to(device)


def moment_sums(n_units: int, d: int, n_evicted, seed: int, device="cpu", s_scale: float = 1.0):
    """Running sums of an evicted set, drawn at the size a sum of n unit-normal rows has:
    n [n_units] int32 (n_evicted, an int or a per-unit list), s_k and s_v [n_units, d]
    ~ sqrt(n) N(0,1), S [n_units, d, d] ~ s_scale sqrt(n) N(0,1); all fp32. They are not
    the sums of any particular rows (every fp32 value is a valid input of the moment model);
    s_scale > 1 makes the key-dependent part of the model as large as the values."""
    n = torch.as_tensor(n_evicted, dtype=torch.int32).expand(n_units).contiguous()
    r = torch.sqrt(n.to(torch.float32))
    sk = _randn((n_units, d), seed, S_MOM, 0, device) * r[:, None].to(device)
    sv = _randn((n_units, d), seed, S_MOM, 1, device) * r[:, None].to(device)
    S = _randn((n_units, d, d), seed, S_MOM, 2, device) * (s_scale * r)[:, None, None].to(device)
    return {"n": n.to(device), "sk": sk, "sv": sv, "S": S}


def token_weights(n_scopes: int, n_slots: int, seed: int, device="cpu", spread: float = 2.0):
    """Positive per-token weights that sum to one per scope, shaped like attention
    weights: exp(spread * N(0,1)) normalised; fp32 [n_scopes, n_slots]."""
    z = torch.exp(spread * _randn((n_scopes, n_slots), seed, S_ALPHA, None, "cpu").double())
    return (z / z.sum(dim=1, keepdim=True)).float().to(device)


def output_projection(n_layers: int, H: int, d: int, D: int, seed: int, device="cpu",
                      std: float = 0.02) -> torch.Tensor:
    """Per-query-head output projection blocks W_O^h: [n_layers, H, d, D] bf16 ~ N(0, std^2)."""
    out = torch.empty((n_layers, H, d, D), dtype=torch.bfloat16, device=device)
    for l in range(n_layers):
        out[l] = (std * _randn((H, d, D), seed, S_WO, l, device)).to(torch.bfloat16)
    return out


def window_queries(n_layers: int, H: int, w: int, d: int, seed: int, device="cpu") -> torch.Tensor:
    """Observation-window queries (the last w prompt positions): [n_layers, H, w, d] bf16 ~ N(0,1)."""
    return _randn((n_layers, H, w, d), seed, S_QWIN, None, device).to(torch.bfloat16)


def laprox_inputs(lw, device="cpu"):
    """Prefill tensors of a LaProx workload: q_win [n_layers, H, w, d], k and v
    [n_layers, n_kv, N, d] (K, V ~ N(0,1) as in kv_rows, unit order
    layer-major), w_o [n_layers, H, d, D] ~ N(0, 0.02^2); all bf16."""
    units = lw.n_layers * lw.n_kv
    k, v = kv_rows(units, lw.N, lw.d, "bf16", lw.seed, device)
    return {"q_win": window_queries(lw.n_layers, lw.H, lw.w, lw.d, lw.seed, device),
            "k": k.view(lw.n_layers, lw.n_kv, lw.N, lw.d), "v": v.view(lw.n_layers, lw.n_kv, lw.N, lw.d),
            "w_o": output_projection(lw.n_layers, lw.H, lw.d, lw.D, lw.seed, device)}


def cache_tensors(wl: Workload, device="cpu", capacity: int | None = None, initial_len: int | None = None):
    """Device tensors of a workload's cache before its first decode step.

    k, v: [n_scopes, units_per_scope, capacity, d] in the cache dtype, the first
    `initial_len` rows drawn as in kv_rows (unit order: scope-major); pos:
    [n_scopes, capacity] int32 (0..L0-1, or a sorted sample of the context when
    the cache starts compressed); m: zeros; length: [n_scopes] int32; votes:
    1 + Poisson(2) when the workload starts from prior merges, else None;
    scales: per-unit key channel scales [n_units, d] or None."""
    cap = capacity or wl.capacity
    L0 = wl.initial_len if initial_len is None else initial_len
    S, U, d = wl.n_scopes, wl.units_per_scope, wl.d
    dt = _DTYPES[wl.dtype]
    scales = key_scales(wl.n_units, d, wl.seed, device) if wl.key_scales else None
    k = torch.zeros((S, U, cap, d), dtype=dt, device=device)
    v = torch.zeros_like(k)
    K0, V0 = kv_rows(wl.n_units, L0, d, wl.dtype, wl.seed, device, scales)
    k[:, :, :L0] = K0.view(S, U, L0, d)
    v[:, :, :L0] = V0.view(S, U, L0, d)
    del K0, V0
    pos = torch.zeros((S, cap), dtype=torch.int32, device=device)
    if wl.prior_votes:
        pos[:, :L0] = initial_positions(S, L0, wl.context, wl.seed, device)
        votes = torch.zeros((S, cap), dtype=torch.int32, device=device)
        votes[:, :L0] = prior_votes(S, L0, wl.seed, device=device)
    else:
        pos[:, :L0] = torch.arange(L0, dtype=torch.int32, device=device)
        votes = None
    m = torch.zeros((S, cap), dtype=torch.float32, device=device)
    length = torch.full((S,), L0, dtype=torch.int32, device=device)
    return {"k": k, "v": v, "pos": pos, "m": m, "length": length, "votes": votes, "scales": scales}


def step_inputs(wl: Workload, step: int, scales=None, device="cpu"):
    """Query heads [n_scopes, units, G, d] and new rows [n_scopes, units, d] of decode step `step` (1-based)."""
    S, U = wl.n_scopes, wl.units_per_scope
    q = step_query(step, wl.n_units, wl.G, wl.d, wl.dtype, wl.seed, device).view(S, U, wl.G, wl.d)
    kn, vn = step_new_kv(step, wl.n_units, wl.d, wl.dtype, wl.seed, device, scales)
    return q, kn.view(S, U, wl.d), vn.view(S, U, wl.d)

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
votes, W_O, window queries, initial positions.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import Workload, WORKLOADS, budget_for  # noqa: F401  (re-export)

S_K, S_V, S_SCALE, S_OUTLIER, S_Q, S_NEWK, S_NEWV, S_VOTES, S_WO, S_QWIN, S_POS = range(11)

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

"""Workload shapes of the fixed-budget decode step and of LaProx prefill scoring.

Shapes only (sizes, dtypes, rules, seeds); no arithmetic of the method. The
budget follows InertiaKV §3: B = floor((1 - rho) * L0), computed in integers
for the 90% compression ratio used by every workload here.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


def budget_for(context: int, keep_tenths: int = 1) -> int:
    """B = floor((1 - rho) L0) with 1 - rho = keep_tenths / 10, in exact integers."""
    return (context * keep_tenths) // 10


@dataclass(frozen=True)
class Workload:
    """One decode-step workload. A *unit* is one KV head of one layer of one
    sequence; a *scope* is the set of units that share one slot set."""
    name: str
    seed: int
    dtype: str            # cache dtype: "bf16" or "f32"
    d: int                # head dimension
    G: int                # query heads per KV head
    n_layers: int
    batch: int
    n_kv: int             # KV heads per layer
    context: int          # L0, live tokens before the first decode step
    budget: int           # B
    steps: int
    rule: str             # "single" | "cumulative" | "ema"
    alpha: float
    scope: str = "kv_head"    # "kv_head" (scope = unit) or "model" (scope = sequence)
    moments: bool = False
    key_scales: bool = False  # per-channel LogNormal key scales with outlier channels
    merge: bool = False       # ZIP-merge the evicted token instead of dropping it
    prior_votes: bool = False # cache starts compressed with votes 1 + Poisson(2)
    lazy_refresh: int = 0     # 0: score every step; R > 0: score on steps with (t-1) % R == 0

    @property
    def n_units(self) -> int:
        return self.n_layers * self.batch * self.n_kv

    @property
    def n_scopes(self) -> int:
        return self.batch if self.scope == "model" else self.n_units

    @property
    def units_per_scope(self) -> int:
        return self.n_layers * self.n_kv if self.scope == "model" else 1

    @property
    def initial_len(self) -> int:
        return self.budget if self.prior_votes else self.context

    @property
    def capacity(self) -> int:
        return self.initial_len + 1

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


@dataclass(frozen=True)
class LaproxWorkload:
    name: str
    seed: int
    n_layers: int
    H: int
    n_kv: int
    d: int
    D: int                # hidden size (columns of W_O)
    N: int                # prompt length
    w: int                # observation window (last w queries)
    keep_per_head: int    # model-wide budget = keep_per_head * n_layers * n_kv

    @property
    def G(self) -> int:
        return self.H // self.n_kv

    @property
    def keep_total(self) -> int:
        return self.keep_per_head * self.n_layers * self.n_kv


WORKLOADS = {
    # Single head, fp32, 4096 cached tokens compressed to 128, 64 steps.
    "c1_head_f32_4k": Workload(
        name="c1_head_f32_4k", seed=1, dtype="f32", d=128, G=1, n_layers=1, batch=1, n_kv=1,
        context=4096, budget=128, steps=64, rule="ema", alpha=0.9, moments=True),
    # One Llama-3.1-8B-shaped layer (32 q / 8 kv heads), 32K context at a 10% budget.
    "c2_llama8b_layer_32k": Workload(
        name="c2_llama8b_layer_32k", seed=2, dtype="bf16", d=128, G=4, n_layers=1, batch=1,
        n_kv=8, context=32768, budget=budget_for(32768), steps=256, rule="ema", alpha=0.9,
        moments=True, key_scales=True),
    # The same layer stacked over the 32 independent layers of the model: one launch per step.
    "c2x32_llama8b_32layers_32k": Workload(
        name="c2x32_llama8b_32layers_32k", seed=22, dtype="bf16", d=128, G=4, n_layers=32,
        batch=1, n_kv=8, context=32768, budget=budget_for(32768), steps=256, rule="ema",
        alpha=0.9, moments=True, key_scales=True),
    # Full Llama-3.1-8B-shaped cache, one slot set per sequence shared by every layer.
    "c3_llama8b_model_16k": Workload(
        name="c3_llama8b_model_16k", seed=3, dtype="bf16", d=128, G=4, n_layers=32, batch=16,
        n_kv=8, context=16384, budget=budget_for(16384), steps=128, rule="ema", alpha=0.8,
        scope="model", key_scales=True),
    # Vote-weighted decode with ZIP merging, cache already at 10% of a 64K context.
    "c4_keepkv_votes_64k": Workload(
        name="c4_keepkv_votes_64k", seed=4, dtype="bf16", d=128, G=4, n_layers=1, batch=8,
        n_kv=8, context=65536, budget=budget_for(65536), steps=64, rule="single", alpha=0.0,
        key_scales=True, merge=True, prior_votes=True),
}
# MomentKV's setting: Llama-3.1-8B (32 layers x 8 KV heads), per-head budget 1024 (the largest
# budget the page reports), a 32K context, moment-informed eviction every decode step.
WORKLOADS["m1_momentkv_llama8b_32layers_b1024"] = Workload(
    name="m1_momentkv_llama8b_32layers_b1024", seed=6, dtype="bf16", d=128, G=4, n_layers=32, batch=1,
    n_kv=8, context=32768, budget=1024, steps=64, rule="single", alpha=0.0, moments=True, key_scales=True)
# KeepKV prefill compression: every KV head of a Llama-3.1-8B-shaped model (32 layers x 8),
# a 4K prompt merged down to 10% by greedy all-pairs ZIP merging, the last 32 positions kept.
WORKLOADS["k1_keepkv_prefill_llama8b_4k"] = Workload(
    name="k1_keepkv_prefill_llama8b_4k", seed=7, dtype="bf16", d=128, G=4, n_layers=32, batch=1, n_kv=8,
    context=4096, budget=budget_for(4096), steps=1, rule="single", alpha=0.0, key_scales=True, merge=True)
WORKLOADS["c3_llama8b_model_16k_lazy8"] = WORKLOADS["c3_llama8b_model_16k"].scaled(
    name="c3_llama8b_model_16k_lazy8", lazy_refresh=8)

LAPROX_WORKLOADS = {
    # Qwen3-8B-shaped prefill: 36 layers, 32 q / 8 kv heads, hidden 4096, 64K prompt.
    "c5_laprox_qwen3_8b_64k": LaproxWorkload(
        name="c5_laprox_qwen3_8b_64k", seed=5, n_layers=36, H=32, n_kv=8, d=128, D=4096,
        N=65536, w=32, keep_per_head=128),
}

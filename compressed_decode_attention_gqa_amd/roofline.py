"""Algorithmic byte and flop counts of the decode step and LaProx scoring.

"Algorithmic" means what the step must move or compute at minimum, not what
the kernels happen to do: the K/V rows every live token contributes, the
per-token utility read and write and score write, the queries and outputs,
the appended rows, at most one moved row per eviction, the evicted rows the
moment fold reads and the read-modify-write of the moment sums. Workspace
traffic (partials, per-token weights kept for the epilogue) is excluded; the
hardware counters measure it separately.
"""
from __future__ import annotations

from dataclasses import dataclass

MI355X_HBM_GBPS = 8000.0          # published HBM3E bandwidth, GB/s
MI355X_BF16_TFLOPS = 2500.0       # published dense bf16 MFMA, TFLOP/s
MI355X_FP32_VALU_TFLOPS = 157.3
MI355X_FP64_VALU_TFLOPS = 78.6
MI355X_FP64_TFLOPS = 78.6          # published dense fp64 MFMA (same rate as the fp64 vector units)


@dataclass(frozen=True)
class StepBytes:
    kv: int
    utility: int
    score: int
    query: int
    output: int
    append: int
    move: int
    fold_rows: int
    moments: int

    @property
    def total(self) -> int:
        return (self.kv + self.utility + self.score + self.query + self.output + self.append + self.move
                + self.fold_rows + self.moments)


def unit_step_bytes(L: int, k: int, G: int, d: int = 128, elem: int = 2, votes: bool = False,
                    moments: bool = True, write_score: bool = True, units_per_scope: int = 1) -> StepBytes:
    """Bytes of one steady decode step for one unit (one KV head) that attends over L
    live entries (the appended one included) and evicts k of them.

    Per-scope arrays (utility, score, positions, votes) are charged to the unit when a
    scope holds one unit; with several units per scope they are split evenly."""
    row = d * elem
    share = 1.0 / units_per_scope
    per_tok_scope = 4 * 2 + (4 if votes else 0)            # utility read + write (+ vote read)
    kv = L * 2 * row
    utility = int(L * per_tok_scope * share)
    score = int(L * 4 * share) if write_score else 0
    query = G * row
    output = G * d * 4 + G * 4                              # o (fp32) and lse
    append = 2 * row + 2 * row + int(12 * share)            # read new rows, write them; pos/vote/m
    move = k * (2 * 2 * row + int(12 * 2 * share))          # at most one moved row per eviction
    fold_rows = k * 2 * row if moments else 0
    mom = (2 * d * d * 4 + 2 * 2 * d * 4 + 2 * 4) if moments else 0
    return StepBytes(kv, utility, score, query, output, append, move, fold_rows, mom)


def keepkv_memory(n_layers: int, heads: int, budget: int, context: int, d: int, elem: int = 2) -> dict:
    """The KeepKV notes' memory table: votes (int32 per entry), EMA state as the page
    sizes it (budget x d x 2 bytes), and the external full KV (context x d x 2 x 2)."""
    return {"votes_bytes": n_layers * heads * budget * 4,
            "ema_state_bytes": n_layers * heads * budget * d * elem,
            "external_kv_bytes": n_layers * heads * context * d * 2 * elem,
            "vote_overhead": 4 / (2 * d * elem),
            "candidate_pairs": budget * budget}


def kv_cache_bytes(n_layers: int, kv_heads: int, d: int, tokens: int, batch: int, elem: int = 2) -> int:
    return n_layers * kv_heads * d * 2 * elem * tokens * batch


def moment_evict_flops(heads: int, L: int, d: int = 128) -> int:
    """Algorithmic flops of one moment-informed eviction round: per head the model
    A = tau S_tilde / n_e and c = v_bar - A k_bar (3 d^2 + 2 d^2), then for every live
    token the contraction A k_j (2 d^2) and the residual and its squared norm (4 d)."""
    return heads * (5 * d * d + L * (2 * d * d + 4 * d))


"""CPU oracle for the fixed-budget decode step and for LaProx prefill scoring.

TEST INFRASTRUCTURE. This package is the plain, slow, fp64 statement of what
the HIP library computes. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it; the product path never does. It shares no
code with the HIP library (compressed_decode_attention_gqa_amd/): the two meet
only in the seeded inputs of synth/.

Every function writes out the definition it follows and cites the page, and
the section or equation on it, that gives that definition:

  * MomentKV (papercache.org summary, arXiv 2606.01563) -- moment statistics,
    moment-informed eviction (§4.2, Algorithm 1 phase 1) and the
    normalisation-corrected output (Algorithm 1, phase 2).
  * InertiaKV (translated article, arXiv 2609.03515) -- head-averaged
    last-query score, single / cumulative / EMA utility, the lazy-refresh
    alternatives and the rank-stability (Jaccard) measure.
  * KeepKV (reading notes, arXiv 2504.09936) -- vote-weighted attention,
    ZIP-merging, prefill compression by greedy all-pairs merging, and the
    window initialisation and bias correction of the EMA score state.
  * LaProx notes ("Reformulating KV Cache Eviction Problem for Long-Context
    LLM Inference", arXiv 2605.07234) -- prefill score, per-layer
    normalisation, model-wide top-K.

Arithmetic is float64 throughout. Inputs in bf16 or fp32 are widened exactly
(convert.py). A library matmul, sort or sum serves as a step where the
definition is that sum; nothing is blocked, fused or reordered beyond it.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: textbook attention, duplicated-token brute force, the eviction
identity o' = (o - A_e v_e)/(1 - A_e), the retained/evicted split, EMA closed
forms, exhaustive subset enumeration, the centred-covariance identity, the
moment model's exactness on affine values under an isotropic evicted set, the
ZIP lossless property (one merge and a whole greedy prefill compression) and
the pages' worked numbers.

Parity unpinned (these follow from readings of the pages, not from printed
values or identities): the new-token utility start value (zero), the lazy
refresh schedule, the ZIP reference query under GQA (group-mean query), and
the group-summed W_O under GQA in LaProx.
"""
from .convert import to_f64, round_to_bf16, round_to_f32  # noqa: F401
from .attention import attend_unit, scope_score  # noqa: F401
from .utility import SINGLE, CUMULATIVE, EMA, RULES, update_utility  # noqa: F401
from .selection import bottom_k, bottom_k_protected, bottom_k_one_at_a_time, top_k_keep  # noqa: F401
from .moments import fold_moments, centred_moments, empty_moments  # noqa: F401
from .moment_correct import corrected_output, evicted_estimates  # noqa: F401
from .moment_evict import moment_residuals, moment_scores, moment_informed_evict  # noqa: F401
from .compaction import compact  # noqa: F401
from .rank_stability import keep_jaccard  # noqa: F401
from .zip_merge import cosine_partner, zip_merge  # noqa: F401
from .keepkv_prefill import prefill_merge, reference_logits  # noqa: F401
from .keepkv_ema_init import window_scores, ema_window_init, predicted_scores  # noqa: F401
from .keepkv_refresh import refresh  # noqa: F401
from .decode_step import ScopeState, StepParams, decode_step  # noqa: F401
from .laprox import (window_column_norms, value_output_norms, laprox_scores,  # noqa: F401
                     laprox_keep)

"""Fixed-budget KV-cache decode step and LaProx prefill scoring on MI355X.

The computation lives in libkvc.so (hand-written HIP for gfx950, C ABI in
include/kvc.h); `kvc` is its ctypes binding (argument marshalling only) and
`roofline` holds the algorithmic byte and flop counts the benchmark prices
against. PyTorch provides device memory and streams only.
"""
from . import kvc  # noqa: F401
from .kvc import (Cache, KvcError, Moments, kvc_compact, kvc_decode_attn_score,  # noqa: F401
                  kvc_decode_step, kvc_ema_update, kvc_laprox_score, kvc_moment_update,
                  kvc_select_evict, merge_desc, workspace)

__all__ = ["kvc", "Cache", "Moments", "KvcError", "kvc_decode_attn_score", "kvc_decode_step",
           "kvc_ema_update", "kvc_select_evict", "kvc_moment_update", "kvc_compact",
           "kvc_laprox_score", "merge_desc", "workspace"]

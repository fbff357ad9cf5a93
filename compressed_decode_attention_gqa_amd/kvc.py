"""ctypes binding of libkvc (include/kvc.h): argument marshalling only.

Every computation runs in the HIP kernels of libkvc.so; this module turns
torch tensors into device pointers and hands them over on the current torch
stream. If the library has not been built, importing the functions works but
the first call raises, naming the missing file: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvc.so")

KVC_OK = 0
KVC_BF16, KVC_F32 = 0, 1
RULES = {"single": 0, "cumulative": 1, "ema": 2}
DTYPES = {torch.bfloat16: KVC_BF16, torch.float32: KVC_F32}

EXPORTED = ("kvc_decode_attn_score", "kvc_ema_update", "kvc_ema_predict", "kvc_select_evict", "kvc_select_evict_protected",
            "kvc_keep_jaccard", "kvc_compact",
            "kvc_moment_update", "kvc_moment_correct", "kvc_moment_evict", "kvc_keepkv_prefill_merge",
            "kvc_keepkv_prefill_merge_marked", "kvc_keepkv_ema_init", "kvc_keepkv_ema_init_marked",
            "kvc_keepkv_refresh", "kvc_keepkv_refresh_marked", "kvc_keepkv_refresh_workspace_size",
            "kvc_laprox_score", "kvc_laprox_score_marked", "kvc_decode_step", "kvc_decode_step_noalloc",
            "kvc_decode_workspace_size", "kvc_decode_plan", "kvc_decode_groups",
            "kvc_select_workspace_size", "kvc_compact_workspace_size", "kvc_moment_evict_workspace_size",
            "kvc_keepkv_prefill_workspace_size", "kvc_keepkv_ema_init_workspace_size",
            "kvc_laprox_workspace_size",
            "kvc_read_probe", "kvc_workspace_status", "kvc_status_string", "kvc_check", "kvc_version")


class KvcError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        super().__init__(f"{fn} failed: {status_string(code)} ({code})")


class _Cache(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("n_scopes", ctypes.c_int32), ("units_per_scope", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("scope_stride", ctypes.c_int64), ("unit_stride", ctypes.c_int64),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("votes", ctypes.c_void_p),
                ("pos", ctypes.c_void_p), ("m", ctypes.c_void_p), ("len", ctypes.c_void_p)]


class _Moments(ctypes.Structure):
    _fields_ = [("n", ctypes.c_void_p), ("sk", ctypes.c_void_p), ("sv", ctypes.c_void_p), ("S", ctypes.c_void_p)]


class _Merge(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("G", ctypes.c_int32), ("scale", ctypes.c_float),
                ("eps", ctypes.c_float), ("reserved", ctypes.c_int32)]


_lib = None
_P, _I, _F, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "kvc_decode_attn_score": (_I, [_P, _P, _P, _I, _P, _I, _F, _P, _P, _P, _I, _P, _SZ, _P]),
    "kvc_decode_step": (_I, [_P, _P, _P, _I, _P, _I, _F, _I, _F, _I, _I, _P, _P, _P, _P, _P, _P,
                             _I, _I, _I, _P, _SZ, _P]),
    "kvc_decode_step_noalloc": (_I, [_P, _P, _P, _I, _P, _I, _F, _I, _F, _I, _I, _P, _P, _P, _P, _P, _P,
                                     _I, _I, _I, _P, _P]),
    "kvc_ema_update": (_I, [_P, _P, _P, _I, _I, _I, _F, _P]),
    "kvc_ema_predict": (_I, [_P, _P, _I, _I, _F, _I, _P, _P]),
    "kvc_select_evict": (_I, [_P, _P, _P, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "kvc_select_evict_protected": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "kvc_keep_jaccard": (_I, [_P, _P, _P, _I, _I, _P, _P]),
    "kvc_moment_update": (_I, [_P, _P, _P, _P]),
    "kvc_compact": (_I, [_P, _P, _P, _P, _SZ, _P]),
    "kvc_moment_correct": (_I, [_P, _I, _P, _I, _I, _F, _P, _P, _P, _P]),
    "kvc_moment_evict": (_I, [_P, _P, _P, _F, _I, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "kvc_keepkv_prefill_merge": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "kvc_keepkv_prefill_merge_marked": (_I, [_P, _P, _I, _I, _P, _P, _P, _P, _SZ, _P, _P, _I]),
    "kvc_keepkv_ema_init": (_I, [_P, _P, _I, _I, _I, _F, _F, _P, _SZ, _P]),
    "kvc_keepkv_ema_init_marked": (_I, [_P, _P, _I, _I, _I, _F, _F, _P, _SZ, _P, _P, _I]),
    "kvc_laprox_score": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P]),
    "kvc_laprox_score_marked": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _P, _P, _I]),
    "kvc_decode_workspace_size": (_SZ, [_P, _I, _I]),
    "kvc_decode_plan": (_I, [_P, _I, _I, _I, _I, _I]),
    "kvc_decode_groups": (_I, [_P, _P, _I, _F, _I, _F, _I, _I, _I, _I, _P, _P, _P, _I, _P, _SZ, _P]),
    "kvc_select_workspace_size": (_SZ, [_I, _I]),
    "kvc_compact_workspace_size": (_SZ, [_P]),
    "kvc_moment_evict_workspace_size": (_SZ, [_P]),
    "kvc_keepkv_prefill_workspace_size": (_SZ, [_P]),
    "kvc_keepkv_ema_init_workspace_size": (_SZ, [_P, _I, _I, _I]),
    "kvc_keepkv_refresh_workspace_size": (_SZ, [_P, _I, _I, _I]),
    "kvc_keepkv_refresh": (_I, [_P, _P, _P, _P, _I, _P, _I, _P, _F, _I, _I, _P, _P, _P, _SZ, _P]),
    "kvc_keepkv_refresh_marked": (_I, [_P, _P, _P, _P, _I, _P, _I, _P, _F, _I, _I, _P, _P, _P, _SZ, _P, _P, _I]),
    "kvc_laprox_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "kvc_read_probe": (_I, [_P, _SZ, _I, _I, _P, _P]),
    "kvc_workspace_status": (_I, [_P, _P]),
    "kvc_status_string": (ctypes.c_char_p, [_I]),
    "kvc_check": (_I, [_P]),
    "kvc_version": (_I, []),
}


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run compressed_decode_attention_gqa_amd/build.py)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(code: int) -> str:
    return lib().kvc_status_string(code).decode()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _check(fn, code):
    if code != KVC_OK:
        raise KvcError(fn, code)


# ------------------------------------------------------------------ descriptors
@dataclass
class Cache:
    """Device cache of one or more scopes, in the layout include/kvc.h describes.

    k, v: [n_scopes, units, capacity, d] (contiguous); votes (optional), pos, m:
    [n_scopes, capacity]; length: [n_scopes] int32."""
    k: torch.Tensor
    v: torch.Tensor
    pos: torch.Tensor
    m: torch.Tensor
    length: torch.Tensor
    votes: torch.Tensor | None = None

    @property
    def n_scopes(self):
        return self.k.shape[0]

    @property
    def units(self):
        return self.k.shape[1]

    @property
    def capacity(self):
        return self.k.shape[2]

    def desc(self) -> _Cache:
        assert self.k.is_contiguous() and self.v.is_contiguous()
        S, U, C, d = self.k.shape
        return _Cache(DTYPES[self.k.dtype], d, C, S, U, 0, U * C, C, _ptr(self.k), _ptr(self.v),
                      _ptr(self.votes), _ptr(self.pos), _ptr(self.m), _ptr(self.length))


@dataclass
class Moments:
    n: torch.Tensor     # [n_scopes, units] int32
    sk: torch.Tensor    # [n_scopes, units, d] f32
    sv: torch.Tensor
    S: torch.Tensor     # [n_scopes, units, d, d] f32

    @staticmethod
    def zeros(n_scopes, units, d=128, device="cuda"):
        return Moments(torch.zeros((n_scopes, units), dtype=torch.int32, device=device),
                       torch.zeros((n_scopes, units, d), device=device),
                       torch.zeros((n_scopes, units, d), device=device),
                       torch.zeros((n_scopes, units, d, d), device=device))

    def desc(self) -> _Moments:
        return _Moments(_ptr(self.n), _ptr(self.sk), _ptr(self.sv), _ptr(self.S))


def merge_desc(q: torch.Tensor, G: int, scale: float, eps: float = 1e-6) -> _Merge:
    return _Merge(_ptr(q), G, scale, eps, 0)


# ------------------------------------------------------------------ entry points
def kvc_decode_workspace_size(cache: Cache, G: int, max_len: int = 0) -> int:
    d = cache.desc()
    return lib().kvc_decode_workspace_size(ctypes.byref(d), G, max_len)


PLAN_ONE_LAUNCH, PLAN_SPLIT, PLAN_SPLIT_BULK = 1, 2, 3


def kvc_decode_plan(cache: Cache, G: int, step: bool = True, merge: bool = False, budget: int = 0,
                    max_len: int = 0) -> int:
    """PLAN_ONE_LAUNCH, PLAN_SPLIT or PLAN_SPLIT_BULK: the kernels kvc_decode_step (step) or
    kvc_decode_attn_score (not step) runs for these shapes."""
    d = cache.desc()
    plan = lib().kvc_decode_plan(ctypes.byref(d), G, int(step), int(merge), budget, max_len)
    if plan < 0:
        raise KvcError("kvc_decode_plan", plan)
    return plan


def kvc_select_workspace_size(n_scopes: int, capacity: int) -> int:
    return lib().kvc_select_workspace_size(n_scopes, capacity)


def kvc_compact_workspace_size(cache: Cache) -> int:
    d = cache.desc()
    return lib().kvc_compact_workspace_size(ctypes.byref(d))


def kvc_moment_evict_workspace_size(cache: Cache) -> int:
    d = cache.desc()
    return lib().kvc_moment_evict_workspace_size(ctypes.byref(d))


def kvc_keepkv_prefill_workspace_size(cache: Cache) -> int:
    d = cache.desc()
    return lib().kvc_keepkv_prefill_workspace_size(ctypes.byref(d))


def kvc_keepkv_ema_init_workspace_size(cache: Cache, G: int, n_win: int, n_tokens: int) -> int:
    d = cache.desc()
    return lib().kvc_keepkv_ema_init_workspace_size(ctypes.byref(d), G, n_win, n_tokens)


def kvc_laprox_workspace_size(n_layers, H, n_kv, N, w, d, D) -> int:
    return lib().kvc_laprox_workspace_size(n_layers, H, n_kv, N, w, d, D)


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (its first word is the device status word)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def kvc_workspace_status(ws: torch.Tensor, stream=None) -> int:
    return lib().kvc_workspace_status(_ptr(ws), _stream(stream))


def kvc_check(stream=None) -> int:
    """Synchronises the stream; 0, or KVC_ERR_DEVICE after an asynchronous device error."""
    return lib().kvc_check(_stream(stream))


def kvc_decode_attn_score(cache: Cache, k_new, v_new, t: int, q, G: int, scale: float, out, lse, s,
                          max_len: int, ws: torch.Tensor, stream=None):
    d = cache.desc()
    _check("kvc_decode_attn_score", lib().kvc_decode_attn_score(
        ctypes.byref(d), _ptr(k_new), _ptr(v_new), t, _ptr(q), G, scale, _ptr(out), _ptr(lse), _ptr(s),
        max_len, _ptr(ws), ws.numel(), _stream(stream)))


def kvc_decode_step(cache: Cache, k_new, v_new, t: int, q, G: int, scale: float, rule, alpha: float,
                    budget: int, out, lse, s=None, moments: Moments | None = None, merge: _Merge | None = None,
                    evict_out=None, refresh: bool = True, attn_unit0: int = 0, attn_units: int = 0,
                    max_len: int = 0, ws: torch.Tensor = None, stream=None):
    d = cache.desc()
    mom = moments.desc() if moments is not None else None
    rule = RULES.get(rule, rule)
    _check("kvc_decode_step", lib().kvc_decode_step(
        ctypes.byref(d), _ptr(k_new), _ptr(v_new), t, _ptr(q), G, scale, rule, alpha, budget, int(refresh),
        _ptr(out), _ptr(lse), _ptr(s), ctypes.byref(mom) if mom is not None else None,
        ctypes.byref(merge) if merge is not None else None, _ptr(evict_out), attn_unit0, attn_units, max_len,
        _ptr(ws), ws.numel(), _stream(stream)))


def kvc_decode_groups(cache: Cache, q, G: int, scale: float, rule, alpha: float, unit0: int, n_groups: int,
                      group_units: int, out, lse, s=None, refresh: bool = True, max_len: int = 0,
                      ws: torch.Tensor = None, stream=None):
    d = cache.desc()
    rule = RULES.get(rule, rule)
    _check("kvc_decode_groups", lib().kvc_decode_groups(
        ctypes.byref(d), _ptr(q), G, scale, rule, alpha, int(refresh), unit0, n_groups, group_units,
        _ptr(out), _ptr(lse), _ptr(s), max_len, _ptr(ws), ws.numel(), _stream(stream)))


def kvc_decode_step_noalloc(cache: Cache, k_new, v_new, t: int, q, G: int, scale: float, rule, alpha: float,
                            budget: int, out, lse, s=None, moments: Moments | None = None,
                            merge: _Merge | None = None, evict_out=None, refresh: bool = True, attn_unit0: int = 0,
                            attn_units: int = 0, max_len: int = 0, status=None, stream=None):
    d = cache.desc()
    mom = moments.desc() if moments is not None else None
    rule = RULES.get(rule, rule)
    _check("kvc_decode_step_noalloc", lib().kvc_decode_step_noalloc(
        ctypes.byref(d), _ptr(k_new), _ptr(v_new), t, _ptr(q), G, scale, rule, alpha, budget, int(refresh),
        _ptr(out), _ptr(lse), _ptr(s), ctypes.byref(mom) if mom is not None else None,
        ctypes.byref(merge) if merge is not None else None, _ptr(evict_out), attn_unit0, attn_units, max_len,
        _ptr(status), _stream(stream)))


def kvc_read_probe(buf: torch.Tensor, workgroups: int, sink: torch.Tensor, reverse: bool = False,
                   nbytes: int | None = None, stream=None):
    nb = buf.numel() * buf.element_size() if nbytes is None else nbytes
    _check("kvc_read_probe", lib().kvc_read_probe(_ptr(buf), nb, workgroups, int(reverse), _ptr(sink),
                                                  _stream(stream)))


def kvc_ema_update(m, s, length, n_scopes: int, capacity: int, rule, alpha: float, stream=None):
    rule = RULES.get(rule, rule)
    _check("kvc_ema_update", lib().kvc_ema_update(_ptr(m), _ptr(s), _ptr(length), n_scopes, capacity, rule,
                                                  alpha, _stream(stream)))


def kvc_select_evict(key, pos, length, n_scopes: int, capacity: int, budget: int, evict, n_evict,
                     ws: torch.Tensor, stream=None):
    _check("kvc_select_evict", lib().kvc_select_evict(
        _ptr(key), _ptr(pos), _ptr(length), n_scopes, capacity, budget, _ptr(evict), _ptr(n_evict),
        _ptr(ws), ws.numel(), _stream(stream)))


def kvc_select_evict_protected(key, pos, length, n_scopes: int, capacity: int, budget: int, protect_from: int,
                               evict, n_evict, ws: torch.Tensor, stream=None):
    _check("kvc_select_evict_protected", lib().kvc_select_evict_protected(
        _ptr(key), _ptr(pos), _ptr(length), n_scopes, capacity, budget, protect_from, _ptr(evict), _ptr(n_evict),
        _ptr(ws), ws.numel(), _stream(stream)))


def kvc_keep_jaccard(keep_a, keep_b, length, n_scopes: int, capacity: int, out, stream=None):
    _check("kvc_keep_jaccard", lib().kvc_keep_jaccard(_ptr(keep_a), _ptr(keep_b), _ptr(length), n_scopes,
                                                      capacity, _ptr(out), _stream(stream)))


def kvc_moment_update(cache: Cache, evict, moments: Moments, stream=None):
    d = cache.desc()
    mom = moments.desc()
    _check("kvc_moment_update", lib().kvc_moment_update(ctypes.byref(d), _ptr(evict), ctypes.byref(mom),
                                                        _stream(stream)))


def kvc_moment_correct(moments: Moments, n_units: int, q, G: int, scale: float, f_R, lse_R, out, stream=None):
    mom = moments.desc()
    dtype = KVC_BF16 if q.dtype == torch.bfloat16 else KVC_F32
    _check("kvc_moment_correct", lib().kvc_moment_correct(ctypes.byref(mom), n_units, _ptr(q), dtype, G, scale,
                                                          _ptr(f_R), _ptr(lse_R), _ptr(out), _stream(stream)))


def kvc_moment_evict(cache: Cache, moments: Moments, alpha, scale: float, budget: int, evict, order=None,
                     score_out=None, n_evict=None, max_len: int = 0, ws: torch.Tensor = None, stream=None):
    d = cache.desc()
    mom = moments.desc()
    _check("kvc_moment_evict", lib().kvc_moment_evict(
        ctypes.byref(d), ctypes.byref(mom), _ptr(alpha), scale, budget, max_len, _ptr(evict), _ptr(order),
        _ptr(score_out), _ptr(n_evict), _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)))


def kvc_keepkv_prefill_merge(cache: Cache, merge: _Merge, budget: int, protect_from: int, evict, pairs=None,
                             n_merged=None, ws: torch.Tensor = None, stream=None, events=None):
    """events: None, or 4 recorded-once torch.cuda.Event(enable_timing=True) objects, re-recorded
    on the launch stream before the first kernel and after each of the three."""
    d = cache.desc()
    nbytes = ws.numel() if ws is not None else 0
    if events is None:
        _check("kvc_keepkv_prefill_merge", lib().kvc_keepkv_prefill_merge(
            ctypes.byref(d), ctypes.byref(merge), budget, protect_from, _ptr(evict), _ptr(pairs), _ptr(n_merged),
            _ptr(ws), nbytes, _stream(stream)))
        return
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("kvc_keepkv_prefill_merge_marked", lib().kvc_keepkv_prefill_merge_marked(
        ctypes.byref(d), ctypes.byref(merge), budget, protect_from, _ptr(evict), _ptr(pairs), _ptr(n_merged),
        _ptr(ws), nbytes, _stream(stream), handles, len(events)))


def kvc_keepkv_refresh_workspace_size(cache: Cache, G: int, n_win: int, n_tokens: int) -> int:
    d = cache.desc()
    return lib().kvc_keepkv_refresh_workspace_size(ctypes.byref(d), G, n_win, n_tokens)


def kvc_keepkv_refresh(cache: Cache, host_k, host_v, host_pos, n_tokens: int, q_win, n_win: int, merge: _Merge,
                       alpha: float, budget: int, protect_from: int, pairs=None, n_merged=None,
                       ws: torch.Tensor = None, stream=None, events=None):
    """host_k, host_v: pinned host tensors [n_scopes, n_tokens, 128] bf16; host_pos: pinned
    [n_scopes, n_tokens] int32. events: None, or 5 recorded-once torch.cuda.Event(enable_timing=True)."""
    for name, t in (("host_k", host_k), ("host_v", host_v), ("host_pos", host_pos)):
        if t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous host tensor")
    d = cache.desc()
    args = (ctypes.byref(d), ctypes.c_void_p(host_k.data_ptr()), ctypes.c_void_p(host_v.data_ptr()),
            ctypes.c_void_p(host_pos.data_ptr()), n_tokens, _ptr(q_win), n_win, ctypes.byref(merge), alpha, budget,
            protect_from, _ptr(pairs), _ptr(n_merged), _ptr(ws), ws.numel(), _stream(stream))
    if events is None:
        _check("kvc_keepkv_refresh", lib().kvc_keepkv_refresh(*args))
        return
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("kvc_keepkv_refresh_marked", lib().kvc_keepkv_refresh_marked(*args, handles, len(events)))


def kvc_keepkv_ema_init(cache: Cache, q_win, G: int, n_win: int, n_tokens: int, scale: float, alpha: float,
                        ws: torch.Tensor, stream=None, events=None):
    """events: None, or 5 recorded-once torch.cuda.Event(enable_timing=True) objects."""
    d = cache.desc()
    if events is None:
        _check("kvc_keepkv_ema_init", lib().kvc_keepkv_ema_init(
            ctypes.byref(d), _ptr(q_win), G, n_win, n_tokens, scale, alpha, _ptr(ws), ws.numel(), _stream(stream)))
        return
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("kvc_keepkv_ema_init_marked", lib().kvc_keepkv_ema_init_marked(
        ctypes.byref(d), _ptr(q_win), G, n_win, n_tokens, scale, alpha, _ptr(ws), ws.numel(), _stream(stream),
        handles, len(events)))


def kvc_ema_predict(m, length, n_scopes: int, capacity: int, alpha: float, t: int, out, stream=None):
    _check("kvc_ema_predict", lib().kvc_ema_predict(_ptr(m), _ptr(length), n_scopes, capacity, alpha, t, _ptr(out),
                                                    _stream(stream)))


def kvc_compact(cache: Cache, evict, merge: _Merge | None, ws: torch.Tensor, stream=None):
    d = cache.desc()
    _check("kvc_compact", lib().kvc_compact(ctypes.byref(d), _ptr(evict),
                                            ctypes.byref(merge) if merge is not None else None,
                                            _ptr(ws), ws.numel(), _stream(stream)))


def kvc_laprox_score(q_win, k, v, w_o, n_layers, H, n_kv, N, w, d, D, scale, score, ws, stream=None,
                     events=None):
    """events: None, or 8 recorded-once torch.cuda.Event(enable_timing=True) objects; they are
    re-recorded on the launch stream around the seven stages."""
    if events is None:
        _check("kvc_laprox_score", lib().kvc_laprox_score(
            _ptr(q_win), _ptr(k), _ptr(v), _ptr(w_o), n_layers, H, n_kv, N, w, d, D, scale, _ptr(score),
            _ptr(ws), ws.numel(), _stream(stream)))
        return
    handles = (ctypes.c_void_p * len(events))(*[e.cuda_event for e in events])
    _check("kvc_laprox_score_marked", lib().kvc_laprox_score_marked(
        _ptr(q_win), _ptr(k), _ptr(v), _ptr(w_o), n_layers, H, n_kv, N, w, d, D, scale, _ptr(score),
        _ptr(ws), ws.numel(), _stream(stream), handles, len(events)))

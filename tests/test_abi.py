"""The C ABI: libkvc.so loads, exports every function include/kvc.h declares, and
rejects bad arguments on the host before enqueuing anything (CPU only: no call
here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from compressed_decode_attention_gqa_amd import kvc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvc.h")

needs_lib = pytest.mark.skipif(not os.path.exists(kvc.LIB_PATH), reason="libkvc.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("kvc_decode_attn_score", "kvc_ema_update", "kvc_select_evict", "kvc_compact",
               "kvc_moment_update", "kvc_laprox_score", "kvc_decode_step"):
        assert fn in names
    assert set(names) == set(kvc.EXPORTED)


@needs_lib
def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(kvc.LIB_PATH)
    for fn in declared_functions():
        assert hasattr(h, fn), fn
    assert kvc.lib().kvc_version() == 1
    assert kvc.status_string(0) == "ok"
    assert kvc.status_string(-6).startswith("workspace")


def _fake_cache(**over):
    fields = dict(dtype=0, head_dim=128, capacity=100, n_scopes=2, units_per_scope=1, reserved=0,
                  scope_stride=100, unit_stride=100, k=0x1000, v=0x2000, votes=None, pos=0x3000, m=0x4000,
                  len=0x5000)
    fields.update(over)
    return kvc._Cache(**fields)


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(head_dim=64), -3), (dict(dtype=5), -2), (dict(k=0x1008), -5), (dict(capacity=0), -1),
    (dict(pos=None), -1), (dict(units_per_scope=2, unit_stride=10), -1)])
def test_decode_step_rejects_bad_cache(over, code):
    c = _fake_cache(**over)
    r = kvc.lib().kvc_decode_step(ctypes.byref(c), None, None, 0, 0x6000, 4, 0.1, 2, 0.9, 10, 1, 0x7000,
                                  0x8000, None, None, None, None, 0, 0, 0, 0x9000, 1 << 30, None)
    assert r == code


@needs_lib
def test_decode_step_host_checks():
    c = _fake_cache()
    L = kvc.lib()
    args = lambda **kw: dict(dict(q=0x6000, G=4, budget=10, max_len=0, ws=0x9000, wsb=1 << 30, kn=None, vn=None), **kw)

    def call(a):
        return L.kvc_decode_step(ctypes.byref(c), a["kn"], a["vn"], 0, a["q"], a["G"], 0.1, 2, 0.9, a["budget"], 1,
                                 0x7000, 0x8000, None, None, None, None, 0, 0, a["max_len"], a["ws"], a["wsb"], None)
    assert call(args(G=3)) == -3
    assert call(args(q=None)) == -1
    assert call(args(q=0x6004)) == -5
    assert call(args(budget=-1)) == -4
    assert call(args(max_len=101)) == -4
    assert call(args(ws=None)) == -6
    assert call(args(wsb=16)) == -6
    assert call(args(kn=0x100)) == -1          # new key without new value
    need = L.kvc_decode_workspace_size(ctypes.byref(c), 4, 0)
    assert need > 0 and L.kvc_decode_workspace_size(ctypes.byref(c), 3, 0) == 0


@needs_lib
def test_decode_plan_host_logic():
    """The plan query: argument errors as the step returns them; a live-length bound above
    budget + 1 takes the bulk kernels without merge and not with it (neither depends on the device)."""
    L = kvc.lib()
    c = _fake_cache()
    plan = lambda G=4, step=1, merge=0, budget=10, max_len=0: L.kvc_decode_plan(ctypes.byref(c), G, step, merge,
                                                                                 budget, max_len)
    assert plan(G=3) == -3
    assert plan(max_len=101) == -4
    assert plan(budget=-1) == -4
    assert plan() == kvc.PLAN_SPLIT_BULK
    assert plan(merge=1) == kvc.PLAN_SPLIT
    bad = _fake_cache(head_dim=64)
    assert L.kvc_decode_plan(ctypes.byref(bad), 4, 1, 0, 10, 0) == -3


@needs_lib
def test_decode_groups_host_checks():
    """kvc_decode_groups rejects a unit range outside the scope, group sizes beyond one call's
    head limit, bad rules, refresh without utilities, null or misaligned pointers and a short
    workspace before enqueuing anything."""
    L = kvc.lib()

    def call(c, q=0x6000, G=4, rule=2, refresh=1, unit0=2, n_groups=3, gu=2, out=0x7000, max_len=0, ws=0x9000,
             wsb=1 << 30):
        return L.kvc_decode_groups(ctypes.byref(c), q, G, 0.1, rule, 0.9, refresh, unit0, n_groups, gu, out, 0x8000,
                                   None, max_len, ws, wsb, None)
    c = _fake_cache(units_per_scope=8, unit_stride=100, scope_stride=800)
    assert call(c, unit0=3) == -1                 # 3 + 3 * 2 > 8 units
    assert call(c, n_groups=0) == -1
    assert call(c, gu=0) == -1
    assert call(c, unit0=-1) == -1
    assert call(c, G=3) == -3
    assert call(c, G=8, gu=16, n_groups=0) == -1
    c1 = _fake_cache(units_per_scope=20, unit_stride=100, scope_stride=2000)
    assert call(c1, G=8, unit0=0, n_groups=1, gu=9) == -3   # 72 heads in one group
    assert call(c, rule=7) == -1
    assert call(c, q=None) == -1
    assert call(c, q=0x6004) == -5
    assert call(c, out=None) == -1
    assert call(c, max_len=101) == -4
    assert call(c, ws=None) == -6
    assert call(c, wsb=16) == -6
    nm = _fake_cache(units_per_scope=8, unit_stride=100, scope_stride=800, m=None)
    assert call(nm) == -1


@needs_lib
def test_keepkv_refresh_host_checks():
    """kvc_keepkv_refresh: per-KV-head bf16 caches with votes and utilities only; window, token count,
    alpha, pointers and workspace checked on the host before anything is enqueued."""
    L = kvc.lib()
    mg = kvc._Merge(q=0x6000, G=4, scale=0.1, eps=1e-6)

    def call(c, hk=0x100, n=50, qw=0x7000, n_win=8, merge=mg, alpha=0.9, budget=10, ws=0x9000, wsb=1 << 30):
        return L.kvc_keepkv_refresh(ctypes.byref(c), hk, 0x200, 0x300, n, qw, n_win,
                                    ctypes.byref(merge) if merge is not None else None, alpha, budget, 40, None, None,
                                    ws, wsb, None)
    c = _fake_cache(votes=0x5100)
    assert call(_fake_cache(votes=0x5100, dtype=1)) == -2
    assert call(_fake_cache(votes=0x5100, units_per_scope=2, unit_stride=100, scope_stride=200)) == -3
    assert call(_fake_cache()) == -1                     # no votes
    assert call(c, hk=None) == -1
    assert call(c, merge=None) == -1
    assert call(c, qw=0x7004) == -5
    assert call(c, alpha=1.0) == -1
    assert call(c, n=101) == -4
    assert call(c, n_win=0) == -4
    assert call(c, n_win=60) == -4
    assert call(c, budget=-1) == -4
    assert call(c, ws=None) == -6
    assert call(c, wsb=16) == -6
    assert L.kvc_keepkv_refresh_workspace_size(ctypes.byref(c), 4, 8, 50) > 0
    assert L.kvc_keepkv_refresh_workspace_size(ctypes.byref(c), 4, 60, 50) == 0


@needs_lib
def test_other_entry_points_reject_bad_arguments():
    L = kvc.lib()
    assert L.kvc_ema_update(None, 0x10, 0x20, 1, 10, 2, 0.9, None) == -1
    assert L.kvc_ema_update(0x10, 0x10, 0x20, 1, 10, 7, 0.9, None) == -1
    assert L.kvc_select_evict(0x10, None, None, 1, 10, -1, 0x20, None, 0x30, 4096, None) == -4
    assert L.kvc_select_evict(0x10, None, None, 1, 10, 3, 0x20, None, None, 0, None) == -6
    c = _fake_cache()
    assert L.kvc_compact(ctypes.byref(c), None, None, 0x30, 1 << 20, None) == -1
    assert L.kvc_moment_update(ctypes.byref(c), 0x10, None, None) == -1
    assert L.kvc_laprox_score(0x10, 0x20, 0x30, 0x40, 1, 32, 8, 100, 4, 64, 4096, 0.1, 0x50, 0x60, 1 << 30,
                              None) == -3
    assert L.kvc_laprox_score(0x10, 0x20, 0x30, 0x40, 1, 30, 8, 100, 4, 128, 4096, 0.1, 0x50, 0x60, 1 << 30,
                              None) == -3
    # KeepKV eq. (14) prediction: 0 < alpha < 1, t >= 1, non-null arrays
    assert L.kvc_ema_predict(None, None, 1, 10, 0.9, 3, 0x10, None) == -1
    assert L.kvc_ema_predict(0x10, None, 1, 10, 0.9, 0, 0x10, None) == -1
    assert L.kvc_ema_predict(0x10, None, 1, 10, 1.0, 3, 0x10, None) == -1
    assert L.kvc_ema_predict(0x10, None, 0, 10, 0.9, 3, 0x10, None) == -1


@needs_lib
def test_merge_needs_votes():
    """A ZIP merge stores p_e + p_c (KeepKV eq. (7)): without a votes array the step and the
    standalone compaction reject merge mode before enqueuing anything."""
    L = kvc.lib()
    mg = kvc._Merge(0x8000, 4, 0.1, 1e-6, 0)
    c = _fake_cache()
    assert L.kvc_compact(ctypes.byref(c), 0x10, ctypes.byref(mg), 0x30, 1 << 30, None) == -1
    r = L.kvc_decode_step(ctypes.byref(c), None, None, 0, 0x6000, 4, 0.1, 0, 0.9, 10, 1, 0x7000, 0x8000, None,
                          None, ctypes.byref(mg), None, 0, 0, 0, 0x9000, 1 << 30, None)
    assert r == -1
    cv = _fake_cache(votes=0x7000)
    assert L.kvc_compact(ctypes.byref(cv), 0x10, ctypes.byref(kvc._Merge(0x8000, 3, 0.1, 1e-6, 0)), 0x30,
                         1 << 30, None) == -1


@needs_lib
def test_moment_evict_host_checks():
    L = kvc.lib()
    mom = kvc._Moments(n=0x100, sk=0x200, sv=0x300, S=0x400)
    c = _fake_cache()
    need = L.kvc_moment_evict_workspace_size(ctypes.byref(c))
    assert need > 0

    def call(cache=c, m=mom, alpha=0x500, budget=10, max_len=0, evict=0x600, ws=0x700, wsb=need):
        return L.kvc_moment_evict(ctypes.byref(cache), ctypes.byref(m) if m is not None else None, alpha, 0.1,
                                  budget, max_len, evict, None, None, None, ws, wsb, None)
    assert call(cache=_fake_cache(units_per_scope=2, unit_stride=100, scope_stride=200)) == -3
    assert call(cache=_fake_cache(head_dim=64)) == -3
    assert call(m=None) == -1
    assert call(m=kvc._Moments(n=0x100, sk=0x200, sv=0x300, S=0x408)) == -5
    assert call(m=kvc._Moments(n=0x100, sk=0x204, sv=0x300, S=0x400)) == -5
    assert call(alpha=None) == -1
    assert call(evict=None) == -1
    assert call(budget=-1) == -4
    assert call(max_len=101) == -4
    assert call(ws=None) == -1
    assert call(wsb=need - 1) == -6


@needs_lib
def test_keepkv_prefill_host_checks():
    L = kvc.lib()
    c = _fake_cache(votes=0x7000)
    mg = kvc._Merge(0x8000, 4, 0.1, 1e-6, 0)
    need = L.kvc_keepkv_prefill_workspace_size(ctypes.byref(c))
    assert need > 0

    def call(cache=c, m=mg, budget=10, evict=0x600, ws=0x900, wsb=need):
        return L.kvc_keepkv_prefill_merge(ctypes.byref(cache), ctypes.byref(m) if m is not None else None, budget,
                                          90, evict, None, None, ws, wsb, None)
    assert call(cache=_fake_cache(votes=0x7000, units_per_scope=2, unit_stride=100, scope_stride=200)) == -3
    big = _fake_cache(votes=0x7000, capacity=32769, scope_stride=32769)
    assert call(cache=big, wsb=L.kvc_keepkv_prefill_workspace_size(ctypes.byref(big))) == -3   # > 32768 slots
    assert call(cache=_fake_cache()) == -1                    # no votes
    assert call(m=None) == -1
    assert call(m=kvc._Merge(0x8000, 3, 0.1, 1e-6, 0)) == -3
    assert call(m=kvc._Merge(0x8008, 4, 0.1, 1e-6, 0)) == -5
    assert call(evict=None) == -1
    assert call(budget=-1) == -4
    assert call(wsb=need - 1) == -6


@needs_lib
def test_keepkv_ema_init_host_checks():
    L = kvc.lib()
    c = _fake_cache()
    need = L.kvc_keepkv_ema_init_workspace_size(ctypes.byref(c), 4, 33, 90)
    assert need > 0

    def call(cache=c, q=0x8000, G=4, n_win=33, n_tok=90, alpha=0.9, wsb=need, ev=None, n_ev=0):
        return L.kvc_keepkv_ema_init_marked(ctypes.byref(cache), q, G, n_win, n_tok, 0.1, alpha, 0x900, wsb,
                                            None, ev, n_ev)
    assert call(cache=_fake_cache(units_per_scope=2, unit_stride=100, scope_stride=200)) == -3
    assert call(G=3) == -3
    assert call(cache=_fake_cache(dtype=1)) == -2              # fp32 caches
    assert call(q=None) == -1
    assert call(cache=_fake_cache(m=None)) == -1
    assert call(alpha=1.0) == -1 and call(alpha=0.0) == -1
    assert call(n_win=0) == -4 and call(n_tok=101) == -4 and call(n_win=91) == -4
    assert call(q=0x8008) == -5
    assert call(wsb=need - 1) == -6
    assert call(ev=(ctypes.c_void_p * 2)(), n_ev=2) == -1     # five events or none


@needs_lib
@pytest.mark.parametrize("H,n_kv,N,w,D,code", [
    (32, 8, 100, 1, 4096, -3),     # G w = 4: not a whole number of 8-row waves
    (32, 8, 100, 4, 4000, -3),     # D not a multiple of 64
    (32, 8, 3, 4, 4096, -3),       # window longer than the prompt
    (48, 8, 100, 4, 4096, -3),     # G = 6
    (32, 8, 100, 4, 4096, 0)])     # supported
def test_laprox_shape_checks(H, n_kv, N, w, D, code):
    L = kvc.lib()
    need = L.kvc_laprox_workspace_size(2, H, n_kv, N, w, 128, D)
    assert (need == 0) == (code != 0)
    if code:
        assert L.kvc_laprox_score(0x10, 0x20, 0x30, 0x40, 2, H, n_kv, N, w, 128, D, 0.1, 0x50, 0x60, 1 << 40,
                                  None) == code
    else:
        # the workspace must cover the layout; pointers are checked first
        assert L.kvc_laprox_score(0x10, 0x20, 0x30, 0x40, 2, H, n_kv, N, w, 128, D, 0.1, 0x50, 0x60, need - 1,
                                  None) == -6
        assert L.kvc_laprox_score(None, 0x20, 0x30, 0x40, 2, H, n_kv, N, w, 128, D, 0.1, 0x50, 0x60, need,
                                  None) == -1
        assert L.kvc_laprox_score(0x18, 0x20, 0x30, 0x40, 2, H, n_kv, N, w, 128, D, 0.1, 0x50, 0x60, need,
                                  None) == -5


@needs_lib
def test_laprox_workspace_covers_the_full_size_prefill():
    # 36 layers x 8 KV heads, N = 65536, w = 32, D = 4096: two float64 Gram halves per unit,
    # the per-token c^2 (one block of 128 window rows) and r^2, the window rows' partials
    need = kvc.kvc_laprox_workspace_size(36, 32, 8, 65536, 32, 128, 4096)
    units = 36 * 8
    assert need >= units * 2 * 128 * 128 * 8 + units * 65536 * 4 + units * 65536 * 4
    assert need < 0.4e9


# ------------------------------------------------------------ host logic: bytes model
def _golden(name):
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", name)):
        line = line.split("#")[0].strip()
        if line:
            rows.append(line.split())
    return rows


def test_keepkv_memory_arithmetic_matches_page_figures():
    """KeepKV notes' memory table worked example (LLaMA-3-8B, 32 layers, 32 heads as
    the page counts them, d = 128, L = 32768, B = 3277) and background KV-size example."""
    from compressed_decode_attention_gqa_amd import roofline as rf
    mem = rf.keepkv_memory(32, 32, 3277, 32768, 128)
    mem["llama70b_kv_bytes"] = rf.kv_cache_bytes(80, 8, 128, 8192, 128) / 2 ** 30
    for name, val, unit, tol in _golden("keepkv_memory_arithmetic.txt"):
        got = mem[name]
        assert abs(got - float(val)) <= float(tol) * float(val), (name, got, val)


def test_budget_floor_matches_printed_budget():
    """InertiaKV §3 budget floor((1 - rho) L0) vs the KeepKV notes' printed B = 3277."""
    import synth
    for L0, B_printed in _golden("inertiakv_budgets.txt"):
        B = synth.budget_for(int(L0))
        assert B == int(L0) // 10 and abs(B - int(B_printed)) <= 1


def test_step_bytes_model():
    from compressed_decode_attention_gqa_amd import roofline as rf
    b = rf.unit_step_bytes(L=3277, k=1, G=4)
    assert b.kv == 3277 * 512
    assert b.moments == 2 * 128 * 128 * 4 + 2 * 2 * 128 * 4 + 8
    assert 1_850_000 < b.total < 1_860_000          # ~566 bytes per cached token


@needs_lib
def test_noalloc_step_rejects_a_cache_beyond_its_scratch():
    """kvc_decode_step_noalloc runs in a 128 MiB per-GPU scratch array: a cache whose decode
    workspace is larger is refused on the host (KVC_ERR_WORKSPACE) before any device call, and
    the usual argument checks come first."""
    L = kvc.lib()

    def call(c, G=4, q=0x6000):
        return L.kvc_decode_step_noalloc(ctypes.byref(c), None, None, 0, q, G, 0.1, 2, 0.9, 10, 1, 0x7000, 0x8000,
                                         None, None, None, None, 0, 0, 0, None, None)
    big = _fake_cache(capacity=1 << 20, n_scopes=256, scope_stride=1 << 20)
    assert L.kvc_decode_workspace_size(ctypes.byref(big), 4, 0) > (128 << 20)
    assert call(big) == -6
    assert call(_fake_cache(head_dim=64)) == -3
    assert call(_fake_cache(), G=3) == -3
    assert call(_fake_cache(k=0x1008)) == -5

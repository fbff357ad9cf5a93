"""GPU parity of InertiaKV's Score-Free limit and of the lazy-refresh alternatives (MI355X).

Score-Free is the lazy rule with scores refreshed at the first step only; the pause variant
runs attention alone between refreshes (the cache grows to B + R) and one refresh step then
scores every entry and evicts R at once; the protect variant keeps the entries appended since
the last refresh and evicts, at every step, the lowest stale utility among the scored ones
(kvc_select_evict_protected). All are driven through the C ABI and compared step by step with
the fp64 oracle on the same pre-state (kvc_parity.check_step). They follow from the readings of
the lazy rule, not from values the pages print: parity unpinned beyond the oracle (the protected
selection itself is pinned to exhaustive enumeration on the CPU and compared bit-exactly here).
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle

import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, check_step, lockstep

pytestmark = pytest.mark.gpu

C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]


def test_decode_step_score_free():
    """Scores at step 1 only: later steps hold the budget with the stale utility, so each
    appended entry (utility 0) is the one evicted."""
    wl = C2.scaled(context=1500, budget=150, steps=10, n_kv=3)
    run = DeviceRun(wl)
    rep = lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)), refresh_for_step=lambda t: t == 1)
    print("score-free", rep, flush=True)


@pytest.mark.parametrize("R", [2, 4])
def test_lazy_pause_until_refresh(R):
    """Attention only between refreshes, then R evictions in one refresh step (the bulk path)."""
    wl = C2.scaled(context=1000, budget=100, steps=1, n_kv=2)
    run = DeviceRun(wl)
    scopes = list(range(wl.n_scopes))
    no_evict = dataclasses.replace(wl, budget=10 ** 9)
    for step in range(1, 3 * R + 2):
        q, kn, vn = run.inputs(step)
        refresh = (step - 1) % R == 0
        pre = run.snapshot(scopes)
        t = run.t
        if refresh:
            run.step(step, q, kn, vn, refresh=True, max_len=0 if step == 1 else wl.budget + R + 1)
        else:
            run.evict.zero_()
            kvc.kvc_decode_attn_score(run.cache, kn, vn, t, q, run.G, run.scale, run.out, run.lse, run.s,
                                      0, run.ws)
            run.t += 1
        torch.cuda.synchronize()
        post = run.snapshot(scopes)
        if refresh:
            check_step(run, scopes, pre, post, q, kn, vn, t, refresh=True)
            assert all(int(x) == wl.budget for x in post["len"])
        else:
            saved, run.wl = run.wl, no_evict
            try:
                check_step(run, scopes, pre, post, q, kn, vn, t, refresh=False)
            finally:
                run.wl = saved
    assert kvc.kvc_workspace_status(run.ws) == 0


def test_select_evict_protected_matches_oracle():
    """Bit-exact evicted sets under (protected, key, pos) with heavy ties, ragged lengths,
    permuted positions, and a scope that must give up protected entries."""
    rng = np.random.default_rng(5)
    S, C = 6, 700
    lens = np.array([700, 650, 1, 0, 300, 120])
    budgets = 100
    key = rng.choice([0.0, 0.5, 1.0, 2.0], size=(S, C)).astype(np.float32)
    pos = np.stack([rng.permutation(C) for _ in range(S)]).astype(np.int32)
    protect_from = 600                 # scope 5: 120 live, most unprotected; scope 0: 100 protected
    kd, pd, ld = (torch.from_numpy(x).cuda() for x in (key, pos, lens.astype(np.int32)))
    evict = torch.full((S, C), 7, dtype=torch.uint8, device="cuda")
    n_ev = torch.zeros(S, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_select_workspace_size(S, C))
    kvc.kvc_select_evict_protected(kd, pd, ld, S, C, budgets, protect_from, evict, n_ev, ws)
    torch.cuda.synchronize()
    ev, ne = evict.cpu().numpy(), n_ev.cpu().numpy()
    for s in range(S):
        L = int(lens[s])
        k = max(0, L - budgets)
        ref = np.zeros(L, dtype=np.uint8)
        ref[oracle.bottom_k_protected(key[s, :L], pos[s, :L], k, protect_from)] = 1
        assert np.array_equal(ev[s, :L], ref) and ne[s] == k, s
    # a bound that protects most entries: some protected ones must go to reach the budget
    kvc.kvc_select_evict_protected(kd, pd, ld, S, C, budgets, 50, evict, n_ev, ws)
    torch.cuda.synchronize()
    ev = evict.cpu().numpy()
    for s in range(S):
        L = int(lens[s])
        ref = np.zeros(L, dtype=np.uint8)
        ref[oracle.bottom_k_protected(key[s, :L], pos[s, :L], max(0, L - budgets), 50)] = 1
        assert np.array_equal(ev[s, :L], ref), s
    # no positions: the slot index orders ties and sets the protection
    kvc.kvc_select_evict_protected(kd, None, ld, S, C, budgets, 400, evict, n_ev, ws)
    torch.cuda.synchronize()
    ev = evict.cpu().numpy()
    for s in range(S):
        L = int(lens[s])
        ref = np.zeros(L, dtype=np.uint8)
        ref[oracle.bottom_k_protected(key[s, :L], np.arange(L), max(0, L - budgets), 400)] = 1
        assert np.array_equal(ev[s, :L], ref), s
    # a bound below every position protects everything: the plain selection again
    kvc.kvc_select_evict_protected(kd, pd, ld, S, C, budgets, 0, evict, n_ev, ws)
    torch.cuda.synchronize()
    ev = evict.cpu().numpy()
    for s in range(S):
        L = int(lens[s])
        ref = np.zeros(L, dtype=np.uint8)
        ref[oracle.bottom_k(key[s, :L], pos[s, :L], max(0, L - budgets))] = 1
        assert np.array_equal(ev[s, :L], ref), s


def test_lazy_protect_unscored():
    """Refresh every R = 3 steps; between refreshes attention alone, then the protected
    selection (entries appended since the last refresh kept), fold and compaction."""
    R = 3
    wl = C2.scaled(context=1000, budget=100, steps=1, n_kv=2)
    run = DeviceRun(wl)
    scopes = list(range(wl.n_scopes))
    S, C = wl.n_scopes, run.cache.capacity
    sel_ws = kvc.workspace(kvc.kvc_select_workspace_size(S, C))
    cmp_ws = kvc.workspace(kvc.kvc_compact_workspace_size(run.cache))
    last_refresh = None
    for step in range(1, 3 * R + 2):
        q, kn, vn = run.inputs(step)
        refresh = (step - 1) % R == 0
        pre = run.snapshot(scopes)
        t = run.t
        if refresh:
            run.step(step, q, kn, vn, refresh=True, max_len=0 if step == 1 else wl.budget + 1)
            last_refresh = t
        else:
            kvc.kvc_decode_attn_score(run.cache, kn, vn, t, q, run.G, run.scale, run.out, run.lse, run.s,
                                      0, run.ws)
            kvc.kvc_select_evict_protected(run.cache.m, run.cache.pos, run.cache.length, S, C, wl.budget,
                                           last_refresh + 1, run.evict, None, sel_ws)
            if run.mom is not None:
                kvc.kvc_moment_update(run.cache, run.evict, run.mom)
            kvc.kvc_compact(run.cache, run.evict, None, cmp_ws)
            run.t += 1
        torch.cuda.synchronize()
        post = run.snapshot(scopes)
        check_step(run, scopes, pre, post, q, kn, vn, t, refresh=refresh,
                   protect_from=None if refresh else last_refresh + 1)
        assert all(int(x) == wl.budget for x in post["len"])
    assert kvc.kvc_workspace_status(run.ws) == 0


def test_keep_jaccard_matches_oracle():
    """The rank-stability diagnostic: random kept sets with ragged lengths (exact counts, so
    the ratio is bit-exact), and the kept sets of two scorers on one decode-step state (the
    step's single-step score s against the EMA utility m, top B of each)."""
    rng = np.random.default_rng(8)
    S, C = 5, 3000
    lens = np.array([3000, 2999, 0, 1, 1777], dtype=np.int32)
    a = (rng.random((S, C)) < 0.3).astype(np.uint8)
    b = (rng.random((S, C)) < 0.7).astype(np.uint8)
    out = torch.zeros(S, dtype=torch.float32, device="cuda")
    kvc.kvc_keep_jaccard(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), torch.from_numpy(lens).cuda(),
                         S, C, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for s in range(S):
        L = int(lens[s])
        assert got[s] == np.float32(oracle.keep_jaccard(a[s, :L], b[s, :L])), s
    kvc.kvc_keep_jaccard(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(), None, S, C, out)   # every slot
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for s in range(S):
        assert got[s] == np.float32(oracle.keep_jaccard(a[s], b[s])), s
    # two scorers on one state
    wl = C2.scaled(context=1000, budget=100, steps=1, n_kv=3)
    run = DeviceRun(wl)
    for step in (1, 2):
        q, kn, vn = run.inputs(step)
        run.step(step, q, kn, vn, refresh=True, max_len=0 if step == 1 else wl.budget + 1)
    q, kn, vn = run.inputs(3)
    kvc.kvc_decode_attn_score(run.cache, kn, vn, run.t, q, run.G, run.scale, run.out, run.lse, run.s, 0, run.ws)
    torch.cuda.synchronize()
    Sn, Cn = wl.n_scopes, run.cache.capacity
    ws = kvc.workspace(kvc.kvc_select_workspace_size(Sn, Cn))
    ev_s = torch.zeros((Sn, Cn), dtype=torch.uint8, device="cuda")
    ev_m = torch.zeros_like(ev_s)
    B2 = wl.budget // 2            # keep half: the two scorers' sets then differ
    kvc.kvc_select_evict(run.s, run.cache.pos, run.cache.length, Sn, Cn, B2, ev_s, None, ws)
    kvc.kvc_select_evict(run.cache.m, run.cache.pos, run.cache.length, Sn, Cn, B2, ev_m, None, ws)
    out = torch.zeros(Sn, dtype=torch.float32, device="cuda")
    kvc.kvc_keep_jaccard(1 - ev_s, 1 - ev_m, run.cache.length, Sn, Cn, out)
    torch.cuda.synchronize()
    L = run.cache.length.cpu().numpy()
    sv, mv, pv = run.s.cpu().numpy(), run.cache.m.cpu().numpy(), run.cache.pos.cpu().numpy()
    got = out.cpu().numpy()
    for s in range(Sn):
        n = int(L[s])
        keep_s = np.ones(n, dtype=bool)
        keep_s[oracle.bottom_k(sv[s, :n], pv[s, :n], n - B2)] = False
        keep_m = np.ones(n, dtype=bool)
        keep_m[oracle.bottom_k(mv[s, :n], pv[s, :n], n - B2)] = False
        assert got[s] == np.float32(oracle.keep_jaccard(keep_s, keep_m)), s
    print("jaccard(single-step score, EMA utility) per KV head:", np.round(got, 4), flush=True)
    assert kvc.kvc_check() == 0

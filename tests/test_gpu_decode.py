"""GPU parity of the fused decode step and the attention entry point (MI355X).

Every test calls the HIP library through the C ABI (ctypes) and compares with
the fp64 oracle on the same bytes; see kvc_parity.py for the bar.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, bits, check_step, f32, lockstep, oracle_state

pytestmark = pytest.mark.gpu

C1 = synth.WORKLOADS["c1_head_f32_4k"]
C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]
C2X32 = synth.WORKLOADS["c2x32_llama8b_32layers_32k"]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype,G,L,votes,layers", [("bf16", 4, 1000, True, 1), ("bf16", 4, 129, False, 1),
                                                     ("f32", 1, 777, False, 1), ("bf16", 1, 300, True, 1),
                                                     ("bf16", 8, 260, False, 1), ("f32", 4, 65, True, 1),
                                                     # 136 scopes: one workgroup per head
                                                     ("bf16", 4, 517, True, 46), ("bf16", 8, 300, False, 46),
                                                     ("f32", 2, 201, False, 46), ("bf16", 1, 90, True, 46)])
def test_attn_score_matches_oracle(dtype, G, L, votes, layers):
    _say("attn_score", dtype, G, L, votes, layers)
    wl = C2.scaled(dtype=dtype, G=G, context=L, budget=L, n_kv=3, n_layers=layers, key_scales=True,
                   prior_votes=False)
    run = DeviceRun(wl, capacity=L + 5)
    if votes:
        run.cache.votes = torch.randint(0, 4, (wl.n_scopes, run.cache.capacity), dtype=torch.int32, device="cuda")
        run.cache.votes[:, 0] = 1
    pre = run.snapshot(list(range(wl.n_scopes)))
    q, kn, vn = run.inputs(1)
    kvc.kvc_decode_attn_score(run.cache, kn, vn, wl.context, q, G, run.scale, run.out, run.lse, run.s, 0, run.ws)
    torch.cuda.synchronize()
    post = run.snapshot(list(range(wl.n_scopes)))
    out, lse, s = bits(run.out), bits(run.lse), bits(run.s)
    for sc in range(wl.n_scopes):
        st = oracle_state(pre, sc, dtype)
        K = np.concatenate([st.K, oracle.to_f64(bits(kn)[sc], dtype)[:, None]], 1)
        V = np.concatenate([st.V, oracle.to_f64(bits(vn)[sc], dtype)[:, None]], 1)
        p = np.append(st.votes, 1)
        _, a, o, l = oracle.attend_unit(oracle.to_f64(bits(q)[sc, 0], dtype), K[0], V[0], p, run.scale)
        tol = 2e-3 if dtype == "bf16" else 1e-5 * np.abs(o).max()
        assert np.abs(out[sc, 0] - o).max() <= tol
        assert np.abs(lse[sc, 0] - l).max() <= (2e-3 if dtype == "bf16" else 1e-5 * np.abs(l).max() + 1e-6)
        s_ref = oracle.scope_score([a])
        assert np.all(np.abs(s[sc, :L + 1] - s_ref) <= 1e-5 * s_ref + 1e-12)
        assert post["len"][sc] == L + 1
        assert post["pos"][sc, L] == wl.context and post["m"][sc, L] == 0
        assert np.array_equal(post["k"][sc][:, L], bits(kn)[sc])
        if votes:
            assert post["votes"][sc, L] == 1


@pytest.mark.parametrize("layers", [1, 46])
def test_attn_score_without_utilities(layers):
    """Attention only, no appended row and no utility array (m = NULL): the per-head kernel
    (46 layers x 3 heads = 138 scopes) and the split kernel read no utilities."""
    _say("attn_score without m", layers)
    L = 400
    wl = C2.scaled(context=L, budget=L, n_kv=3, n_layers=layers, key_scales=True, prior_votes=False)
    run = DeviceRun(wl, capacity=L + 3)
    pre = run.snapshot(list(range(wl.n_scopes)))
    run.cache.m = None
    q, _, _ = run.inputs(1)
    kvc.kvc_decode_attn_score(run.cache, None, None, 0, q, wl.G, run.scale, run.out, run.lse, run.s, L,
                              run.ws)
    torch.cuda.synchronize()
    out, lse, s = bits(run.out), bits(run.lse), bits(run.s)
    for sc in range(0, wl.n_scopes, 7):
        st = oracle_state(pre, sc, "bf16")
        _, a, o, l = oracle.attend_unit(oracle.to_f64(bits(q)[sc, 0], "bf16"), st.K[0], st.V[0], st.votes,
                                        run.scale)
        assert np.abs(out[sc, 0] - o).max() <= 2e-3
        assert np.abs(lse[sc, 0] - l).max() <= 2e-3
        s_ref = oracle.scope_score([a])
        assert np.all(np.abs(s[sc, :L] - s_ref) <= 1e-5 * s_ref + 1e-12)
    assert np.all(run.cache.length.cpu().numpy() == L)


@pytest.mark.parametrize("plan", ["one_launch", "split"])
def test_decode_step_c1_lockstep(plan):
    """Single fp32 head, 4096 tokens to a 128 budget, 64 steps, every step checked. one_launch: the
    steady steps bound the live length by budget + 1, so the library runs them as one launch of
    the per-scope kernel (129 rows of 512 bytes per scope); split: no bound (split-K attention and
    the score/finish kernels every step)."""
    run = DeviceRun(C1)
    if plan == "one_launch":
        ml = lambda t: C1.context + 1 if t == 1 else C1.budget + 1
        assert kvc.kvc_decode_plan(run.cache, C1.G, budget=C1.budget, max_len=C1.budget + 1) == kvc.PLAN_ONE_LAUNCH
    else:
        ml = lambda t: None
        assert kvc.kvc_decode_plan(run.cache, C1.G, budget=C1.budget) == kvc.PLAN_SPLIT_BULK
    rep = lockstep(run, C1.steps, lambda t: [0], max_len_for_step=ml)
    _say("c1", plan, rep)


def test_decode_plan_choice():
    """Steady steps of single-unit scopes run as one launch with >= 128 scopes or <= 256 KiB of rows
    per scope; a literal C2 layer (8 heads of 3277 bf16 rows, 1.7 MB each) keeps split-K; a larger
    live-length bound without merge adds the bulk eviction kernels, with merge it does not."""
    c1 = DeviceRun(C1.scaled(context=300, budget=128, steps=1))
    assert kvc.kvc_decode_plan(c1.cache, 1, budget=128, max_len=129) == kvc.PLAN_ONE_LAUNCH
    assert kvc.kvc_decode_plan(c1.cache, 1, step=False, max_len=129) == kvc.PLAN_ONE_LAUNCH
    assert kvc.kvc_decode_plan(c1.cache, 1, budget=128, max_len=301) == kvc.PLAN_SPLIT_BULK
    c2 = DeviceRun(C2.scaled(steps=1))
    B = C2.budget
    assert kvc.kvc_decode_plan(c2.cache, 4, budget=B, max_len=B + 1) == kvc.PLAN_SPLIT
    assert kvc.kvc_decode_plan(c2.cache, 4, budget=B, max_len=C2.context + 1) == kvc.PLAN_SPLIT_BULK
    assert kvc.kvc_decode_plan(c2.cache, 4, budget=B, merge=True, max_len=C2.context + 1) == kvc.PLAN_SPLIT
    c2x = DeviceRun(C2.scaled(n_layers=16, context=B + 8, steps=1))
    assert kvc.kvc_decode_plan(c2x.cache, 4, budget=B, max_len=B + 1) == kvc.PLAN_ONE_LAUNCH


def test_decode_step_c2_reduced_lockstep():
    wl = C2.scaled(context=2000, budget=200, steps=12)
    run = DeviceRun(wl)
    rep = lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)))
    _say("c2 reduced", rep)


@pytest.mark.parametrize("rule", ["single", "cumulative"])
def test_decode_step_other_rules(rule):
    wl = C2.scaled(context=1500, budget=300, steps=5, rule=rule, n_kv=4)
    run = DeviceRun(wl)
    lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)))


def test_decode_step_lazy_refresh():
    wl = C2.scaled(context=1200, budget=1100, steps=9, n_kv=2)
    run = DeviceRun(wl)
    lockstep(run, wl.steps, lambda t: [0, 1], refresh_for_step=lambda t: (t - 1) % 4 == 0)


def test_decode_step_c2_full_size():
    """One Llama-3.1-8B layer, 32768 -> 3276 at step 1 (29493 evictions per head), then steady steps."""
    run = DeviceRun(C2, max_len=C2.context + 1)
    checked = {1, 2, 3, 16}
    rep = lockstep(run, 16, lambda t: list(range(C2.n_scopes)) if t in checked else [])
    _say("c2 full", rep)


def test_decode_step_c2x32_sampled():
    """The 32-layer stack in one launch per step at the benchmark's launch shape (step 1 bulk
    compression over 32769 tokens per head, then steady steps with max_len = budget + 1, which
    take the one-workgroup-per-head kernel); sampled scopes."""
    rng = np.random.default_rng(5)
    run = DeviceRun(C2X32, max_len=C2X32.context + 1)

    def scopes(t):
        if t in (1, 2, 3, 8):
            return sorted(rng.choice(C2X32.n_scopes, size=24, replace=False).tolist())
        return []
    rep = lockstep(run, 8, scopes, max_len_for_step=lambda t: None if t == 1 else C2X32.budget + 1)
    _say("c2x32", rep)


@pytest.mark.parametrize("dtype,G,votes,rule", [("bf16", 4, False, "ema"), ("bf16", 4, True, "single"),
                                                ("f32", 1, False, "ema"), ("bf16", 2, True, "cumulative"),
                                                ("bf16", 8, False, "ema")])
def test_decode_step_per_head_kernel(dtype, G, votes, rule):
    """Enough single-head scopes (136) and a short cache: steady steps run one workgroup per head."""
    wl = C2.scaled(dtype=dtype, G=G, n_layers=17, context=700, budget=130, steps=5, rule=rule,
                   key_scales=dtype == "bf16", prior_votes=votes)
    if votes:
        wl = wl.scaled(budget=wl.context // 10 * 9)
    run = DeviceRun(wl, max_len=wl.initial_len + 1)
    assert wl.n_scopes >= 128
    # step 1 compresses in bulk (split kernel); later steps evict one entry each
    rep = lockstep(run, wl.steps, lambda t: list(range(0, wl.n_scopes, 3)),
                   max_len_for_step=lambda t: None if t == 1 else wl.budget + 1)
    _say("per-head", dtype, G, votes, rule, rep)


@pytest.mark.parametrize("path", ["split", "per_head"])
def test_determinism(path):
    """Two runs of the same steps leave bit-identical caches (rows, utilities, positions, moment
    sums) and give bit-identical lse and scores: the normalisers and per-token weights are summed
    in a fixed order. The per-head kernel hands sub-chunks to its waves in run-dependent order,
    which orders the value sums, so its outputs may differ in their last bits (checked to 1e-6)."""
    if path == "split":
        wl, ml = C2.scaled(context=900, budget=100, steps=3, n_kv=3), lambda t: None
    else:
        wl = C2.scaled(n_layers=17, context=900, budget=100, steps=5)
        ml = lambda t: wl.context + 1 if t == 1 else wl.budget + 1
    states = []
    for _ in range(2):
        run = DeviceRun(wl, max_len=wl.context + 1)
        for step in range(1, wl.steps + 1):
            run.step(step, *run.inputs(step), max_len=ml(step))
        torch.cuda.synchronize()
        L = int(run.cache.length.max())
        states.append([bits(x) for x in (run.cache.k, run.cache.v, run.cache.m[:, :L], run.cache.pos[:, :L],
                                         run.mom.S, run.mom.sk, run.lse, run.s[:, :L + 1])] + [bits(run.out)])
    for a, b in zip(states[0][:-1], states[1][:-1]):
        assert np.array_equal(a, b)
    oa, ob = states[0][-1].astype(np.float64), states[1][-1].astype(np.float64)
    assert np.all(np.abs(oa - ob) <= 1e-6 * np.abs(oa).max(axis=-1, keepdims=True))


def test_empty_cache_and_within_budget():
    wl = C2.scaled(context=0, budget=5, steps=7, n_kv=2, moments=True)
    run = DeviceRun(wl, capacity=8)
    lockstep(run, wl.steps, lambda t: [0, 1])


def test_capacity_overflow_is_reported():
    wl = C2.scaled(context=10, budget=20, n_kv=1)
    run = DeviceRun(wl, capacity=11)
    run.step(1, *run.inputs(1))          # fills the last slot
    run.step(2, *run.inputs(2))          # no slot left: device status
    assert kvc.kvc_workspace_status(run.ws) == -4
    assert int(run.cache.length[0]) == 11
    assert kvc.kvc_workspace_status(run.ws) == 0


def test_select_evict_matches_oracle():
    rng = np.random.default_rng(3)
    n_scopes, cap = 5, 3000
    ws = kvc.workspace(kvc.kvc_select_workspace_size(n_scopes, cap))
    for trial in range(4):
        vals = rng.choice(np.array([0.0, 1e-3, 2.5e-3, 7.0, 1e-40], dtype=np.float32), size=(n_scopes, cap))
        vals = np.where(rng.random((n_scopes, cap)) < 0.5, rng.random((n_scopes, cap)).astype(np.float32), vals)
        pos = np.stack([rng.permutation(100000)[:cap] for _ in range(n_scopes)]).astype(np.int32)
        lens = rng.integers(1, cap + 1, size=n_scopes).astype(np.int32)
        budget = int(rng.integers(0, cap))
        key = torch.from_numpy(vals).cuda()
        evict = torch.zeros((n_scopes, cap), dtype=torch.uint8, device="cuda")
        nev = torch.zeros(n_scopes, dtype=torch.int32, device="cuda")
        kvc.kvc_select_evict(key, torch.from_numpy(pos).cuda(), torch.from_numpy(lens).cuda(), n_scopes, cap,
                             budget, evict, nev, ws)
        ev = bits(evict)
        for s in range(n_scopes):
            L = lens[s]
            E = oracle.bottom_k(vals[s, :L].astype(np.float64), pos[s, :L], L - budget)
            assert np.array_equal(np.flatnonzero(ev[s, :L]), E)
            assert int(bits(nev)[s]) == max(0, L - budget)


def test_select_evict_device_wide_top_k():
    """One scope of 2^21 flattened scores keeping the top 4096 (LaProx model-wide Top-K form)."""
    rng = np.random.default_rng(11)
    n, K = 1 << 21, 4096
    vals = rng.random(n).astype(np.float32) ** 3
    vals[rng.choice(n, 5000, replace=False)] = vals[7]          # a heavy tie
    key = torch.from_numpy(vals).cuda()
    evict = torch.empty(n, dtype=torch.uint8, device="cuda")
    ws = kvc.workspace(kvc.kvc_select_workspace_size(1, n))
    kvc.kvc_select_evict(key, None, None, 1, n, K, evict, None, ws)
    keep = bits(evict) == 0
    ref = oracle.top_k_keep(vals.astype(np.float64), K)
    assert np.array_equal(keep, ref)


# ---------------------------------------------------------------- KeepKV: votes and ZIP merge
C4 = synth.WORKLOADS["c4_keepkv_votes_64k"]


@pytest.mark.parametrize("flags", [True, False])
@pytest.mark.parametrize("dtype,G,budget", [("bf16", 4, 300), ("f32", 2, 300), ("bf16", 4, 700)])
def test_decode_step_c4_merge_reduced(dtype, G, budget, flags):
    """Vote-weighted decode with a ZIP merge every step (KeepKV eqs. (7)-(12)), every scope checked.
    The f32 case drives some single-step utilities to ~1e-59, below float32's range: they are
    stored as float32 but ranked on their float64 values, as the oracle ranks them. 300 bf16
    rows per scope take the one-launch kernel, the others the split path; without the flags
    output the split path's merge kernels take the selection themselves."""
    _say("c4 reduced", dtype, G, budget, flags)
    wl = C4.scaled(batch=1, n_kv=5, context=3000, budget=budget, steps=10, dtype=dtype, G=G)
    run = DeviceRun(wl, flags=flags)
    rep = lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)), merge=True)
    _say("c4 reduced", dtype, G, budget, flags, rep)
    assert rep.get("merged_rows_exact", 0) > 0


@pytest.mark.parametrize("flags", [True, False])
def test_decode_step_c4_full_size_sampled(flags):
    """64 scopes of 6553 voted entries (10% of 64K), a merge every step for the workload's 64
    steps; 12 sampled scopes checked at the first step and every 8th (without the flags output
    as the bench runs it, and with it)."""
    rng = np.random.default_rng(9)
    run = DeviceRun(C4, flags=flags)
    rep = lockstep(run, C4.steps, lambda t: sorted(rng.choice(C4.n_scopes, 12, replace=False).tolist())
                   if t == 1 or t % 8 == 0 else [], merge=True)
    _say("c4 full", rep)
    assert rep.get("merged_rows_exact", 0) > 0


def test_step_longer_than_the_launch_bound():
    """Full steps with moments on the split path whose device length (1001) passes the launch's
    live-length bound (max_len 600): the per-head score kernel covers the chunks past each
    workgroup's first as it goes and the finish reads the candidates past those it requests at
    entry (G = 8: 256-token chunks, 3 requested of 4). The first step compresses 3000 -> 1000
    with the bound unset. Lockstep against the oracle, every scope."""
    wl = C2.scaled(context=3000, budget=1000, n_kv=4, G=8, moments=True, steps=4)
    run = DeviceRun(wl)
    assert kvc.kvc_decode_plan(run.cache, wl.G, budget=wl.budget, max_len=600) == kvc.PLAN_SPLIT
    rep = lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)),
                   max_len_for_step=lambda t: None if t == 1 else 600)
    _say("step past the launch bound", rep)


@pytest.mark.parametrize("flags", [True, False])
def test_merge_step_longer_than_the_launch_bound(flags):
    """ZIP-merge steps on the split path with the device length (1001) past the live-length bound
    the launch is sized for (max_len 600): the score kernel's workgroups cover the chunks past
    their first as they go, and the merge kernels read the candidates past those they load at
    entry (G = 8: 256-token chunks, 3 loaded of 4). Lockstep against the oracle, every scope."""
    wl = C4.scaled(batch=1, n_kv=3, context=3000, budget=1000, steps=4, G=8)
    run = DeviceRun(wl, flags=flags)
    assert kvc.kvc_decode_plan(run.cache, wl.G, budget=wl.budget, merge=True, max_len=600) == kvc.PLAN_SPLIT
    rep = lockstep(run, wl.steps, lambda t: list(range(wl.n_scopes)), merge=True, max_len_for_step=lambda t: 600)
    _say("merge past the launch bound", flags, rep)


def test_merge_step_that_merges_nothing():
    """Merge-mode steps on the split path that merge nothing (700 bf16 rows per scope): with the
    live length after the append at most the budget the token is appended and nothing merges;
    more than one entry over the budget reports KVC_ERR_UNSUPPORTED and keeps every entry (a
    merge removes one per step); an append into a full cache reports KVC_ERR_CAPACITY and
    leaves the cache as it was. The same with and without the flags output (the finish kernel's
    bookkeeping, or the merge kernels' own), bit for bit."""
    wl = C4.scaled(batch=1, n_kv=3, context=3000, budget=700, steps=1, G=4)
    S = wl.n_scopes
    for budget, capacity, status in ((702, None, 0), (698, None, -3), (690, 700, -4)):
        states = []
        for flags in (True, False):
            run = DeviceRun(wl, capacity=capacity, flags=flags)
            L0 = int(run.cache.length[0])
            assert L0 == 700
            assert kvc.kvc_decode_plan(run.cache, wl.G, budget=budget, merge=True) == kvc.PLAN_SPLIT
            pre = run.snapshot(list(range(S)))
            q, kn, vn = run.inputs(1)
            kvc.kvc_decode_step(run.cache, kn, vn, run.t, q, wl.G, run.scale, wl.rule, run.alpha, budget, run.out,
                                run.lse, run.s, None, kvc.merge_desc(q, wl.G, run.scale), run.evict, ws=run.ws)
            assert kvc.kvc_workspace_status(run.ws) == status, (budget, flags)
            post = run.snapshot(list(range(S)))
            L = L0 if status == -4 else L0 + 1
            assert np.all(post["len"] == L), (budget, flags)
            for key in ("k", "v"):
                assert np.array_equal(post[key][:, :, :L0], pre[key][:, :, :L0]), (budget, flags, key)
            assert np.array_equal(post["pos"][:, :L0], pre["pos"][:, :L0])
            assert np.array_equal(post["votes"][:, :L0], pre["votes"][:, :L0])
            if L > L0:
                assert np.array_equal(post["k"][:, 0, L0], bits(kn)[:, 0]) and np.all(post["pos"][:, L0] == run.t)
                assert np.all(post["votes"][:, L0] == 1)
            states.append([post[key] for key in ("len", "k", "v", "pos", "votes", "m")])
        for a, b in zip(*states):
            assert np.array_equal(a, b), budget


def test_merge_keeps_the_reference_output():
    """KeepKV's single-step check: after the merge, attention of the reference (group-mean)
    query over the merged cache equals attention over the unmerged cache with the new token."""
    wl = C4.scaled(batch=1, n_kv=3, context=2000, budget=200, steps=1, G=4)
    run = DeviceRun(wl)
    q, kn, vn = run.inputs(1)
    qbar = q.float().mean(dim=2, keepdim=True).to(q.dtype).contiguous()     # [S, 1, 1, d]
    # reference output on the unmerged cache: append only (attend, no eviction)
    snap = DeviceRun(wl)
    out0 = torch.empty((wl.n_scopes, 1, 1, wl.d), device="cuda")
    lse0 = torch.empty((wl.n_scopes, 1, 1), device="cuda")
    kvc.kvc_decode_attn_score(snap.cache, kn, vn, snap.t, qbar, 1, run.scale, out0, lse0, None, 0, snap.ws)
    run.step(1, q, kn, vn, merge=kvc.merge_desc(q, run.G, run.scale))
    out1 = torch.empty_like(out0)
    lse1 = torch.empty_like(lse0)
    kvc.kvc_decode_attn_score(run.cache, None, None, run.t, qbar, 1, run.scale, out1, lse1, None, 0, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(run.cache.length, snap.cache.length - 1)
    # lossless in exact arithmetic for the mean logit; here the query is its bf16 rounding and
    # the merged rows are rounded to bf16
    assert (out1 - out0).abs().max().item() <= 2e-3
    assert (lse1 - lse0).abs().max().item() <= 2e-3


# ---------------------------------------------------------------- model scope (InertiaKV)
C3 = synth.WORKLOADS["c3_llama8b_model_16k"]


def _c3_step(run, step, q, kn, vn, refresh, max_len=None, later_within_budget=False, fused=False):
    """One decode step of a model-scope cache: layer by layer, each layer's KV heads attend,
    score (mean over the layer's query heads), update the shared utility and evict; the new
    token's rows of every layer are appended by the first layer's call. later_within_budget:
    the layers after the first are called with budget = capacity (they cannot evict, the first
    layer having evicted to the budget), which lets the library skip their finish launch.
    fused: the first layer's call, then one kvc_decode_groups call for all the later layers."""
    wl = run.wl
    S = wl.n_scopes
    out_l = torch.empty((S, wl.n_kv, run.G, wl.d), device="cuda")
    lse_l = torch.empty((S, wl.n_kv, run.G), device="cuda")
    for l in range(1 if fused else wl.n_layers):
        u0 = l * wl.n_kv
        kvc.kvc_decode_step(run.cache, kn if l == 0 else None, vn if l == 0 else None, run.t,
                            q[:, u0:u0 + wl.n_kv].contiguous(), run.G, run.scale, wl.rule, run.alpha,
                            run.cache.capacity if (later_within_budget and l > 0) else wl.budget,
                            out_l, lse_l, run.s, run.mom, None, run.evict if l == 0 else None, refresh=refresh,
                            attn_unit0=u0, attn_units=wl.n_kv, max_len=max_len or 0, ws=run.ws)
        run.out[:, u0:u0 + wl.n_kv] = out_l
        run.lse[:, u0:u0 + wl.n_kv] = lse_l
    if fused and wl.n_layers > 1:
        nu = (wl.n_layers - 1) * wl.n_kv
        out_g = torch.empty((S, nu, run.G, wl.d), device="cuda")
        lse_g = torch.empty((S, nu, run.G), device="cuda")
        kvc.kvc_decode_groups(run.cache, q[:, wl.n_kv:].contiguous(), run.G, run.scale, wl.rule, run.alpha,
                              wl.n_kv, wl.n_layers - 1, wl.n_kv, out_g, lse_g, run.s, refresh=refresh,
                              max_len=max_len or 0, ws=run.ws)
        run.out[:, wl.n_kv:] = out_g
        run.lse[:, wl.n_kv:] = lse_g
    run.t += 1


def _c3_check(run, scopes, pre, post, q, kn, vn, t, refresh):
    wl = run.wl
    dtype = wl.dtype
    prm = oracle.StepParams(scale=run.scale, rule=wl.rule, alpha=run.alpha, budget=wl.budget,
                            groups=wl.n_layers, score=refresh, row_dtype=dtype)
    idx = torch.as_tensor(scopes, device="cuda")
    out, lse, s_gpu = bits(run.out[idx]), bits(run.lse[idx]), bits(run.s[idx])
    qh, knh, vnh = bits(q), bits(kn), bits(vn)
    worst = 0.0
    for j, sc in enumerate(scopes):
        st = oracle_state(pre, j, dtype)
        post_ref, res = oracle.decode_step(st, oracle.to_f64(knh[sc], dtype), oracle.to_f64(vnh[sc], dtype), t,
                                           oracle.to_f64(qh[sc], dtype), prm)
        assert np.abs(out[j] - res.o).max() <= 2e-3 and np.abs(lse[j] - res.lse).max() <= 2e-3
        Lp = int(post["len"][j])
        assert Lp == post_ref.length
        ppos = post["pos"][j, :Lp].astype(np.int64)
        assert sorted(ppos.tolist()) == sorted(post_ref.pos.tolist()), f"scope {sc}: surviving positions"
        # the last layer's scores over the final live set
        if refresh:
            s_ref = res.s[-1]
            s_pos = res.s_pos[-1]
            got = {int(p): float(v) for p, v in zip(ppos, s_gpu[j, :Lp])}
            for p, v in zip(s_pos.tolist(), s_ref.tolist()):
                if p in got:
                    assert abs(got[p] - v) <= 1e-5 * abs(v) + 1e-12, f"scope {sc}: s at pos {p}"
        m_ref = dict(zip(post_ref.pos.tolist(), post_ref.m.tolist()))
        pm = post["m"][j, :Lp].astype(np.float64)
        dm = np.array([abs(a - m_ref[int(p)]) / (abs(m_ref[int(p)]) + 1e-30) for a, p in zip(pm, ppos)])
        worst = max(worst, float(dm.max()))
        assert np.all(dm <= 1e-5 + 1e-12), f"scope {sc}: utilities"
        slot_of = {p: i for i, p in enumerate(st.pos.tolist())}
        for i, p in enumerate(ppos.tolist()):
            if p == t:
                assert np.array_equal(post["k"][j][:, i], knh[sc]) and np.array_equal(post["v"][j][:, i], vnh[sc])
            else:
                assert np.array_equal(post["k"][j][:, i], pre["k"][j][:, slot_of[p]])
    return worst


@pytest.mark.parametrize("fused", [False, True])
@pytest.mark.parametrize("lazy", [0, 3])
def test_decode_step_c3_model_scope_reduced(lazy, fused):
    """One slot set per sequence shared by every layer: score and evict after each layer
    (fused: the layers after the first in one kvc_decode_groups call, utility chain in closed form)."""
    wl = C3.scaled(n_layers=4, batch=2, n_kv=3, context=700, budget=70, steps=7, lazy_refresh=lazy)
    run = DeviceRun(wl)
    worst = 0.0
    for step in range(1, wl.steps + 1):
        q, kn, vn = run.inputs(step)
        refresh = lazy == 0 or (step - 1) % lazy == 0
        scopes = list(range(wl.n_scopes))
        pre = run.snapshot(scopes)
        t = run.t
        _c3_step(run, step, q, kn, vn, refresh, fused=fused)
        torch.cuda.synchronize()
        worst = max(worst, _c3_check(run, scopes, pre, run.snapshot(scopes), q, kn, vn, t, refresh))
    assert kvc.kvc_workspace_status(run.ws) == 0
    _say("c3 reduced lazy=%d fused=%d: max rel dm %.2e" % (lazy, fused, worst))


@pytest.mark.parametrize("path", ["per_unit", "split"])
@pytest.mark.parametrize("dtype,G,rule,votes", [("bf16", 4, "ema", False), ("f32", 2, "cumulative", True),
                                                ("bf16", 8, "single", False), ("bf16", 1, "ema", True)])
def test_decode_groups_matches_per_layer_calls(dtype, G, rule, votes, path):
    """kvc_decode_groups against the per-layer calls it stands for (budget = capacity, so no
    eviction), on the same state: outputs and lse within float32 summation-order differences,
    the last group's scores, and the utility chain (float64 closed form stored once, against a
    float32 store after every layer) within 1e-6 relative. per_unit: one workgroup per unit
    (a capacity whose per-token state fits in LDS); split: a capacity of 12000 slots, beyond
    LDS, so the call runs split-K attention, the combine and the score kernel."""
    _say("groups vs per layer", dtype, G, rule, votes, path)
    wl = C3.scaled(n_layers=6, batch=3, n_kv=2, context=500, budget=500, steps=1, dtype=dtype, G=G, rule=rule,
                   prior_votes=votes, key_scales=dtype == "bf16")
    cap = 12000 if path == "split" else None
    runs = [DeviceRun(wl, capacity=cap), DeviceRun(wl, capacity=cap)]
    q, _, _ = runs[0].inputs(1)
    nk, S, cap = wl.n_kv, wl.n_scopes, runs[0].cache.capacity
    unit0, n_groups = nk, wl.n_layers - 1
    qg = q[:, unit0:].contiguous()
    outs = [torch.empty((S, n_groups * nk, G, wl.d), device="cuda") for _ in range(2)]
    lses = [torch.empty((S, n_groups * nk, G), device="cuda") for _ in range(2)]
    r0 = runs[0]
    for j in range(n_groups):
        u0 = unit0 + j * nk
        o = torch.empty((S, nk, G, wl.d), device="cuda")
        ls = torch.empty((S, nk, G), device="cuda")
        kvc.kvc_decode_step(r0.cache, None, None, r0.t, q[:, u0:u0 + nk].contiguous(), G, r0.scale, rule, r0.alpha,
                            cap, o, ls, r0.s, None, None, None, attn_unit0=u0, attn_units=nk, ws=r0.ws)
        outs[0][:, j * nk:(j + 1) * nk] = o
        lses[0][:, j * nk:(j + 1) * nk] = ls
    r1 = runs[1]
    kvc.kvc_decode_groups(r1.cache, qg, G, r1.scale, rule, r1.alpha, unit0, n_groups, nk, outs[1], lses[1], r1.s,
                          ws=r1.ws)
    torch.cuda.synchronize()
    oa, ob = outs[0].double(), outs[1].double()
    assert ((oa - ob).abs() <= 1e-6 * oa.abs().amax(dim=-1, keepdim=True) + 1e-30).all()
    assert ((lses[0].double() - lses[1].double()).abs() <= 1e-6 * lses[0].double().abs() + 1e-6).all()
    L = int(r0.cache.length[0])
    for x, y in ((r0.s[:, :L], r1.s[:, :L]), (r0.cache.m[:, :L], r1.cache.m[:, :L])):
        xd, yd = x.double(), y.double()
        assert ((xd - yd).abs() <= 1e-6 * xd.abs() + 1e-30).all()
    assert kvc.kvc_workspace_status(r1.ws) == 0


def test_model_scope_calls_that_cannot_evict_leave_the_same_state():
    """Layers after the first called with budget = capacity (no finish launch) give bit-identical
    outputs, scores, utilities and slots to calls with the real budget, from the bulk first step on."""
    wl = C3.scaled(n_layers=4, batch=3, n_kv=2, context=900, budget=90, steps=5)
    runs = [DeviceRun(wl), DeviceRun(wl)]
    scopes = list(range(wl.n_scopes))
    for step in range(1, wl.steps + 1):
        q, kn, vn = runs[0].inputs(step)
        for flag, run in zip((False, True), runs):
            _c3_step(run, step, q, kn, vn, True, later_within_budget=flag)
        torch.cuda.synchronize()
        a, b = runs[0].snapshot(scopes), runs[1].snapshot(scopes)
        for key in ("len", "k", "v", "pos", "m"):
            assert np.array_equal(a[key], b[key]), (step, key)
        for x, y in ((runs[0].out, runs[1].out), (runs[0].lse, runs[1].lse), (runs[0].s, runs[1].s)):
            assert np.array_equal(bits(x), bits(y)), step
    assert kvc.kvc_workspace_status(runs[1].ws) == 0


# ---------------------------------------------------------------- the entry points composed
@pytest.mark.parametrize("context,budget,steps,n_kv", [(900, 90, 4, 5), (32768, 3276, 2, 8)])
def test_entry_points_compose_to_the_step(context, budget, steps, n_kv):
    """attn_score -> ema_update -> select_evict -> moment_update -> compact equals the oracle's
    step (and the fused step's checks); the second case is one full Llama-3.1-8B layer, whose
    first step evicts 29493 entries per head through the standalone calls."""
    wl = C2.scaled(context=context, budget=budget, steps=steps, n_kv=n_kv, moments=True)
    run = DeviceRun(wl)
    sel_ws = kvc.workspace(kvc.kvc_select_workspace_size(wl.n_scopes, run.cache.capacity))
    cmp_ws = kvc.workspace(kvc.kvc_compact_workspace_size(run.cache))
    n_ev = torch.zeros(wl.n_scopes, dtype=torch.int32, device="cuda")
    rep = {}
    for step in range(1, wl.steps + 1):
        q, kn, vn = run.inputs(step)
        scopes = list(range(wl.n_scopes))
        pre = run.snapshot(scopes)
        t = run.t
        c = run.cache
        kvc.kvc_decode_attn_score(c, kn, vn, t, q, run.G, run.scale, run.out, run.lse, run.s, 0, run.ws)
        kvc.kvc_ema_update(c.m, run.s, c.length, wl.n_scopes, c.capacity, wl.rule, run.alpha)
        run.evict.zero_()
        kvc.kvc_select_evict(c.m, c.pos, c.length, wl.n_scopes, c.capacity, wl.budget, run.evict, n_ev, sel_ws)
        kvc.kvc_moment_update(c, run.evict, run.mom)
        kvc.kvc_compact(c, run.evict, None, cmp_ws)
        run.t += 1
        torch.cuda.synchronize()
        check_step(run, scopes, pre, run.snapshot(scopes), q, kn, vn, t, report=rep)
        assert np.array_equal(n_ev.cpu().numpy(), bits(run.evict).sum(axis=1).astype(np.int32))
    _say("composed", rep)


@pytest.mark.parametrize("path", ["per_layer", "groups_split", "groups_per_unit"])
def test_decode_step_c3_full_size_sampled(path):
    """16 sequences x 32 layers x 8 KV heads sharing one slot set per sequence, 16384 -> 1638:
    the bulk first step and two steady steps, one sequence checked against the oracle. groups_*:
    layers 2-32 in one kvc_decode_groups call; groups_per_unit bounds the steady steps' live
    length by budget + 1 (one workgroup per unit), groups_split does not (split-K attention)."""
    fused = path != "per_layer"
    run = DeviceRun(C3)
    for step in range(1, 4):
        q, kn, vn = run.inputs(step)
        scopes = [5] if step in (1, 3) else []
        if scopes:
            pre = run.snapshot(scopes)
        t = run.t
        ml = C3.budget + 1 if (path == "groups_per_unit" and step > 1) else None
        _c3_step(run, step, q, kn, vn, True, fused=fused, max_len=ml)
        if scopes:
            torch.cuda.synchronize()
            worst = _c3_check(run, scopes, pre, run.snapshot(scopes), q, kn, vn, t, True)
            _say("c3 full step %d %s: max rel dm %.2e" % (step, path, worst))
    assert int(run.cache.length.min()) == C3.budget == int(run.cache.length.max())
    assert kvc.kvc_workspace_status(run.ws) == 0


@pytest.mark.parametrize("dtype,placement", [("f32", "random"), ("bf16", "random"), ("bf16", "ends")])
def test_compact_merge_standalone_matches_oracle(dtype, placement):
    """kvc_compact in merge mode (KeepKV eqs. (7), (10), (12)) on inputs far from underflow:
    per scope the flagged entry is merged into its largest-cosine partner (oracle
    cosine_partner, zip_merge on the group-mean logits), rows within one ulp of the oracle's
    rounded rows, votes and utilities add, every other row keeps its bits; a scope with two
    flagged entries is left untouched and the workspace status reports KVC_ERR_UNSUPPORTED.
    Scope rows of 520 flag bytes start 8 bytes off a 16-byte boundary every other scope, so
    the flag scan's 16-byte middle and byte-wise ends both run; "ends" puts the flags on the
    first slot, the last slot and slot 9, and scope 3's two flags on its first and last."""
    _say("compact merge", dtype, placement)
    rng = np.random.default_rng(21)
    S, cap, G, d = 4, 520, 4, 128
    lens = np.array([500, 333, 2, 480], dtype=np.int32)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    K = torch.from_numpy(rng.standard_normal((S, 1, cap, d)).astype(np.float32)).to(tdt).cuda()
    V = torch.from_numpy(rng.standard_normal((S, 1, cap, d)).astype(np.float32)).to(tdt).cuda()
    votes = torch.from_numpy(rng.integers(1, 5, (S, cap)).astype(np.int32)).cuda()
    pos = torch.from_numpy(np.stack([rng.permutation(10000)[:cap] for _ in range(S)]).astype(np.int32)).cuda()
    m = torch.from_numpy(rng.random((S, cap)).astype(np.float32)).cuda()
    length = torch.from_numpy(lens).cuda()
    cache = kvc.Cache(k=K, v=V, pos=pos, m=m, length=length, votes=votes)
    q = torch.from_numpy(rng.standard_normal((S, 1, G, d)).astype(np.float32)).to(tdt).cuda()
    evict = torch.zeros((S, cap), dtype=torch.uint8, device="cuda")
    if placement == "ends":
        flagged = [0, int(lens[1]) - 1, min(9, int(lens[2]) - 1), 0]
    else:
        flagged = [int(rng.integers(0, L)) for L in lens]
    for s, e in enumerate(flagged):
        evict[s, e] = 1
    second = int(lens[3]) - 1 if placement == "ends" else (flagged[3] + 7) % lens[3]
    evict[3, second] = 1                               # two flags: unsupported, scope untouched
    scale = f32(1 / np.sqrt(d))
    pre = {k: bits(x) for k, x in (("k", K), ("v", V), ("votes", votes), ("pos", pos), ("m", m))}
    ws = kvc.workspace(kvc.kvc_compact_workspace_size(cache))
    kvc.kvc_compact(cache, evict, kvc.merge_desc(q, G, scale), ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_status(ws) == -3
    assert kvc.kvc_workspace_status(ws) == 0
    post = {k: bits(x) for k, x in (("k", K), ("v", V), ("votes", votes), ("pos", pos), ("m", m))}
    plen = length.cpu().numpy()
    qh = oracle.to_f64(bits(q), dtype)
    for s in range(S):
        L = int(lens[s])
        if s == 3:
            assert plen[s] == L
            for key in pre:
                assert np.array_equal(pre[key][s], post[key][s]), key
            continue
        assert plen[s] == L - 1
        Kh = oracle.to_f64(pre["k"][s, 0, :L], dtype)
        Vh = oracle.to_f64(pre["v"][s, 0, :L], dtype)
        e = flagged[s]
        c = oracle.cosine_partner(Kh, e, pre["pos"][s, :L])
        lbar = (scale * (qh[s, 0] @ Kh.T)).mean(axis=0)
        k_r, v_r, p_r, _ = oracle.zip_merge(Kh[e], Vh[e], pre["votes"][s, e], lbar[e], Kh[c], Vh[c],
                                            pre["votes"][s, c], lbar[c])
        ppos = post["pos"][s, :L - 1].tolist()
        assert sorted(ppos) == sorted(set(pre["pos"][s, :L].tolist()) - {int(pre["pos"][s, e])})
        ic = ppos.index(int(pre["pos"][s, c]))
        ulp = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -23
        for got, want in ((post["k"][s, 0, ic], k_r), (post["v"][s, 0, ic], v_r)):
            want_r = oracle.to_f64(oracle.round_to_bf16(want), "bf16") if dtype == "bf16" else \
                oracle.round_to_f32(want).astype(np.float64)
            assert np.all(np.abs(oracle.to_f64(got, dtype) - want_r) <= np.abs(want_r) * ulp + 1e-30)
        assert int(post["votes"][s, ic]) == p_r
        assert abs(float(post["m"][s, ic]) - (float(pre["m"][s, c]) + float(pre["m"][s, e]))) <= 1e-6
        slot_of = {int(p): i for i, p in enumerate(pre["pos"][s, :L].tolist())}
        for i, p in enumerate(ppos):
            if i == ic:
                continue
            j = slot_of[p]
            assert np.array_equal(post["k"][s, 0, i], pre["k"][s, 0, j])
            assert np.array_equal(post["v"][s, 0, i], pre["v"][s, 0, j])
            assert post["votes"][s, i] == pre["votes"][s, j] and post["m"][s, i] == pre["m"][s, j]


@pytest.mark.parametrize("path", ["per_head", "split"])
def test_weights_below_float32_range_rank_as_float64(path):
    """A key of large norm along the step's group-mean query, planted at slot 0 (so the streaming
    meets it first), puts every other logit some 280 below the maximum: their weights and
    single-step utilities (~1e-120) lie below float32's range. They are stored as float32 zeros
    but ranked on their float64 values (InertiaKV §3.1: lowest utility first), so each step evicts
    what the float64 oracle evicts. per_head: 136 scopes at one eviction each (one workgroup per
    head); split: 8 scopes (split-K attention and the score/finish kernels)."""
    _say("underflow ranking", path)
    n = 400 if path == "per_head" else 600     # split: 601 rows of 512 bytes, beyond one launch's 256 KiB
    wl = C2.scaled(n_layers=17 if path == "per_head" else 1, n_kv=8, context=n, budget=n, steps=4,
                   rule="single", key_scales=True)
    run = DeviceRun(wl, max_len=wl.budget + 1, moments=False)
    want = kvc.PLAN_ONE_LAUNCH if path == "per_head" else kvc.PLAN_SPLIT
    assert kvc.kvc_decode_plan(run.cache, wl.G, budget=wl.budget, max_len=wl.budget + 1) == want
    rep = {}
    for step in range(1, wl.steps + 1):
        q, kn, vn = run.inputs(step)
        qbar = q.float().mean(dim=2)                                    # [S, U, d]
        run.cache.k[:, 0, 0] = (100.0 * qbar[:, 0]).to(run.cache.k.dtype)
        scopes = list(range(0, wl.n_scopes, 3 if path == "per_head" else 1))
        pre = run.snapshot(scopes)
        t = run.t
        run.step(step, q, kn, vn)
        torch.cuda.synchronize()
        check_step(run, scopes, pre, run.snapshot(scopes), q, kn, vn, t, report=rep)
        # the weights really left float32's range: most stored utilities are zero
        m = run.cache.m[scopes].cpu().numpy()[:, :wl.budget]
        assert (m == 0).mean() > 0.5
    assert kvc.kvc_workspace_status(run.ws) == 0
    _say("underflow ranking", path, rep)


def test_per_head_kernel_exact_ties_go_by_position():
    """The per-head kernel (136 scopes, one eviction each) on a step that does not refresh scores
    (lazy refresh: the stale utilities rank, the appended entry has 0): several utilities preset
    exactly equal and lowest -- a negative value, +0 and -0 beside the appended entry's 0, a
    negative value below float32's normal range -- so the eviction is the lowest position among
    the tied entries (oracle bottom_k). Checked exactly: the near-tie band would accept any of them."""
    _say("per-head exact ties")
    wl = C2.scaled(n_layers=17, n_kv=8, context=300, budget=300, steps=2, key_scales=True)
    run = DeviceRun(wl, max_len=wl.budget + 1)
    assert wl.n_scopes >= 128
    run.step(1, *run.inputs(1))        # one steady step first: slots no longer in position order
    rng = np.random.default_rng(31)
    m = run.cache.m.cpu().numpy().copy()
    L = int(run.cache.length[0])
    for sc in range(wl.n_scopes):
        J = rng.choice(L, size=int(rng.integers(2, 7)), replace=False)
        kind = sc % 4
        if kind == 0:
            m[sc, J] = -0.25
        elif kind == 1:
            m[sc, J] = np.where(np.arange(len(J)) % 2 == 0, 0.0, -0.0)   # tie the appended entry's 0
        elif kind == 2:
            m[sc, J] = -1e-40                                           # float32 subnormal
        else:
            m[sc, J[:1]] = -1.0                                         # a single lowest entry
    run.cache.m.copy_(torch.from_numpy(m))
    pos = run.cache.pos.cpu().numpy()
    q, kn, vn = run.inputs(2)
    scopes = list(range(wl.n_scopes))
    pre = run.snapshot(scopes)
    t = run.t
    run.step(2, q, kn, vn, refresh=False)
    torch.cuda.synchronize()
    ev = bits(run.evict)
    for sc in scopes:
        mm = np.append(m[sc, :L].astype(np.float64), 0.0)
        pp = np.append(pos[sc, :L].astype(np.int64), t)
        E = oracle.bottom_k(mm, pp, 1)
        got = np.flatnonzero(ev[sc, :L + 1])
        assert got.tolist() == E.tolist(), (sc, got, E, mm[E], pp[E])
    check_step(run, scopes, pre, run.snapshot(scopes), q, kn, vn, t, refresh=False)
    assert kvc.kvc_workspace_status(run.ws) == 0

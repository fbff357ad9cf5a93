"""GPU parity of InertiaKV's Score-Free limit and of the pause-until-refresh lazy variant (MI355X).

Score-Free is the lazy rule with scores refreshed at the first step only; the pause variant
runs attention alone between refreshes (the cache grows to B + R) and one refresh step then
scores every entry and evicts R at once. Both are driven through the C ABI and compared step by
step with the fp64 oracle on the same pre-state (kvc_parity.check_step). They follow from the
readings of the lazy rule, not from values the pages print: parity unpinned beyond the oracle.
"""
import dataclasses

import pytest
import torch

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

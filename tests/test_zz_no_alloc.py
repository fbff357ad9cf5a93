"""kvc_decode_step_noalloc (the decode step on the library's own per-GPU scratch array) against
kvc_decode_step (caller workspace) through the C ABI, on identical caches: three calls in a row,
each later one smaller than the one before (a bulk first step over 136 heads, a steady step of
those heads on the one-workgroup-per-head kernel, then a 3-head cache on the split path), so
every call starts from the scratch contents the previous one left. Results must be bit-identical
(the same kernels run on the same inputs); the caller's status word reports a capacity overflow.
"""
import numpy as np
import pytest
import torch

import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, bits

pytestmark = pytest.mark.gpu

C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]


def _say(*a):
    print(*a, flush=True)


def _noalloc_step(run, step, q, kn, vn, max_len, status):
    kvc.kvc_decode_step_noalloc(run.cache, kn, vn, run.t, q, run.G, run.scale, run.wl.rule, run.alpha,
                                run.wl.budget, run.out, run.lse, run.s, run.mom, None, run.evict,
                                max_len=max_len, status=status)
    run.t += 1


def _assert_same(ra, rb, what):
    ca, cb = ra.cache, rb.cache
    assert torch.equal(ca.length, cb.length), what
    L = int(ca.length.max())
    for name in ("k", "v"):
        assert np.array_equal(bits(getattr(ca, name)), bits(getattr(cb, name))), (what, name)
    for x, y in ((ca.pos, cb.pos), (ca.m, cb.m)):
        assert np.array_equal(bits(x[:, :L]), bits(y[:, :L])), what
    for x, y in ((ra.out, rb.out), (ra.lse, rb.lse)):
        assert np.array_equal(bits(x), bits(y)), what
    # s and the flags are written for the slots live during the step (one more than after it)
    Ls = min(L + 1, ca.capacity)
    assert np.array_equal(bits(ra.s[:, :Ls]), bits(rb.s[:, :Ls])), what
    assert np.array_equal(bits(ra.evict[:, :Ls]), bits(rb.evict[:, :Ls])), what
    if ra.mom is not None:
        for x, y in ((ra.mom.n, rb.mom.n), (ra.mom.sk, rb.mom.sk), (ra.mom.sv, rb.mom.sv), (ra.mom.S, rb.mom.S)):
            assert np.array_equal(bits(x), bits(y)), what


def test_noalloc_matches_workspace_step():
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wl1 = C2.scaled(n_layers=17, n_kv=8, context=700, budget=70, steps=2)       # 136 heads
    ra, rb = DeviceRun(wl1, max_len=wl1.context + 1), DeviceRun(wl1, max_len=wl1.context + 1)
    for step, max_len in ((1, wl1.context + 1), (2, wl1.budget + 1)):
        _say("noalloc call", step, "heads", wl1.n_scopes, "max_len", max_len)
        q, kn, vn = ra.inputs(step)
        ra.step(step, q, kn, vn, max_len=max_len)
        _noalloc_step(rb, step, q, kn, vn, max_len, status)
        torch.cuda.synchronize()
        _assert_same(ra, rb, f"136 heads, step {step}")
    assert int(ra.cache.length.max()) == wl1.budget
    wl2 = C2.scaled(n_kv=3, context=300, budget=290, steps=1)                    # 3 heads
    ra, rb = DeviceRun(wl2), DeviceRun(wl2)
    _say("noalloc call 3 heads", wl2.n_scopes)
    q, kn, vn = ra.inputs(1)
    ra.step(1, q, kn, vn)
    _noalloc_step(rb, 1, q, kn, vn, 0, status)
    torch.cuda.synchronize()
    _assert_same(ra, rb, "3 heads")
    assert int(status.item()) == 0
    assert kvc.kvc_workspace_status(ra.ws) == 0


def test_noalloc_reports_capacity_overflow_in_the_status_word():
    _say("noalloc capacity overflow")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    wl = C2.scaled(context=10, budget=20, n_kv=1)
    run = DeviceRun(wl, capacity=11)
    for step in (1, 2):            # the first call fills the last slot, the second finds none
        q, kn, vn = run.inputs(step)
        _noalloc_step(run, step, q, kn, vn, 0, status)
    torch.cuda.synchronize()
    assert int(status.item()) == -4
    assert int(run.cache.length[0]) == 11


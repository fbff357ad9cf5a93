"""Decode steps replayed from a captured HIP graph (what a serving loop does to take host
submission out of a latency-bound step): the library's calls enqueue kernels only (no
allocation, no memset, no host synchronisation), so a captured sequence of steps, replayed,
must leave the cache exactly as the same steps called one by one.

Two caches start identical. K steps (their own inputs and positions) are captured on one; then,
three times, the same K steps run eagerly on the other and the graph is replayed, with unrelated
eager work and synchronisations in between, and the two caches and outputs are compared bit for
bit after every replay. Shapes: the one-launch kernel (136 scopes), the split path with its score
and finish kernels (one 32K layer, reduced), and the ZIP-merge step on the split path without the
flags output (the merge kernels select).
"""
import numpy as np
import pytest
import torch

import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, bits

pytestmark = pytest.mark.gpu

C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]
C4 = synth.WORKLOADS["c4_keepkv_votes_64k"]
K = 4

CASES = {
    "one_launch": C2.scaled(context=600, budget=150, n_kv=8, n_layers=17, moments=False),
    "split": C2.scaled(context=6000, budget=1500, n_kv=4, moments=True),
    "split_merge": C4.scaled(batch=1, n_kv=3, context=3000, budget=700, G=4),
}


def _state(run):
    c = run.cache
    return [bits(x) for x in (c.k, c.v, c.pos, c.m, c.length, run.out, run.lse, run.s)] + (
        [bits(c.votes)] if c.votes is not None else []) + (
        [bits(run.mom.S), bits(run.mom.sk), bits(run.mom.n)] if run.mom is not None else [])


@pytest.mark.parametrize("case", list(CASES))
def test_graph_replay_matches_eager_steps(case):
    wl = CASES[case]
    print("graph replay", case, flush=True)
    ra, rb = DeviceRun(wl, flags=False), DeviceRun(wl, flags=False)
    merge = wl.merge
    plan = kvc.kvc_decode_plan(ra.cache, wl.G, budget=wl.budget, merge=merge, max_len=wl.budget + 1)
    assert plan == (kvc.PLAN_ONE_LAUNCH if case == "one_launch" else kvc.PLAN_SPLIT)
    # the first step (compression to the budget) eagerly on both
    for r in (ra, rb):
        q, kn, vn = r.inputs(1)
        mg = kvc.merge_desc(q, r.G, r.scale) if merge else None
        kvc.kvc_decode_step(r.cache, kn, vn, r.t, q, r.G, r.scale, wl.rule, r.alpha, wl.budget, r.out, r.lse,
                            r.s, r.mom, mg, None, max_len=wl.initial_len + 1, ws=r.ws)
        r.t += 1
    torch.cuda.synchronize()
    t0 = ra.t
    inputs = [ra.inputs(2 + j) for j in range(K)]
    merges = [kvc.merge_desc(q, wl.G, ra.scale) if merge else None for q, _, _ in inputs]

    def steps(r):
        for j, (q, kn, vn) in enumerate(inputs):
            kvc.kvc_decode_step(r.cache, kn, vn, t0 + j, q, r.G, r.scale, wl.rule, r.alpha, wl.budget, r.out,
                                r.lse, r.s, r.mom, merges[j], None, max_len=wl.budget + 1, ws=r.ws)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):           # captured on torch's side stream, the calls' current stream
        steps(rb)
    torch.cuda.synchronize()
    noise = torch.randn(1 << 20, device="cuda")
    for replay in range(3):
        steps(ra)
        torch.cuda.synchronize()
        noise.mul_(1.0001).add_(float(replay))     # unrelated eager work between the replays
        g.replay()
        torch.cuda.synchronize()
        sa, sb = _state(ra), _state(rb)
        for i, (x, y) in enumerate(zip(sa, sb)):
            assert np.array_equal(x, y), f"{case}: replay {replay}, array {i} differs from the eager steps"
        assert int(ra.cache.length.min()) == wl.budget
    assert kvc.kvc_workspace_status(ra.ws) == 0 and kvc.kvc_workspace_status(rb.ws) == 0

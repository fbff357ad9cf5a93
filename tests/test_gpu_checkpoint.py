"""Checkpoint and resume of the decode state: T steps in one run against T/2 steps, a save of every
state tensor to bytes (torch.save, loaded back with weights_only=True into fresh device
allocations and a fresh workspace), then the remaining T/2 steps. The state a step reads and
writes is the cache (rows, votes, positions, utilities, lengths), the moment sums and the next
position; nothing else carries over between steps, so the two runs end in the same state.

Checked as the determinism test checks two runs: caches, moment sums, lse and scores bit-identical;
outputs within 1e-6 of their row maximum (the per-head kernel orders its value sums by the order
its waves claim sub-chunks)."""
import io

import numpy as np
import pytest
import torch

import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, bits

pytestmark = pytest.mark.gpu

C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]
C4 = synth.WORKLOADS["c4_keepkv_votes_64k"]

CASES = {
    # one workgroup per head (>= 128 scopes, one eviction per step), moment fold
    "per_head": (C2.scaled(n_layers=17, context=900, budget=100, steps=8), False),
    # split attention with the score/finish kernels
    "split": (C2.scaled(context=900, budget=100, steps=6, n_kv=3), False),
    # vote-weighted cache with a ZIP merge every step
    "merge": (C4.scaled(batch=1, n_kv=5, context=3000, budget=300, steps=6, G=4), True),
}


def _run_max_len(wl, path):
    return 0 if path == "merge" else wl.context + 1


def _max_len(wl, path, step):
    if path == "per_head":
        return wl.context + 1 if step == 1 else wl.budget + 1
    return None


def _step(run, wl, path, step, merge):
    q, kn, vn = run.inputs(step)
    run.step(step, q, kn, vn, merge=kvc.merge_desc(q, run.G, run.scale) if merge else None,
             max_len=_max_len(wl, path, step))


def _save(run) -> bytes:
    c, m = run.cache, run.mom
    state = {"k": c.k, "v": c.v, "pos": c.pos, "m": c.m, "length": c.length, "t": torch.tensor(run.t)}
    if c.votes is not None:
        state["votes"] = c.votes
    if m is not None:
        state.update(n=m.n, sk=m.sk, sv=m.sv, S=m.S)
    buf = io.BytesIO()
    torch.save({k: v.detach().cpu() for k, v in state.items()}, buf)
    return buf.getvalue()


def _restore(wl, path, blob: bytes) -> DeviceRun:
    st = torch.load(io.BytesIO(blob), weights_only=True)
    run = DeviceRun(wl, max_len=_run_max_len(wl, path))
    dev = run.cache.k.device
    g = {k: v.to(dev).clone() for k, v in st.items() if k != "t"}
    run.cache = kvc.Cache(k=g["k"], v=g["v"], pos=g["pos"], m=g["m"], length=g["length"], votes=g.get("votes"))
    run.mom = kvc.Moments(g["n"], g["sk"], g["sv"], g["S"]) if "n" in g else None
    run.ws = kvc.workspace(kvc.kvc_decode_workspace_size(run.cache, wl.G, run.max_len), dev)
    run.t = int(st["t"])
    return run


def _state(run):
    torch.cuda.synchronize()
    L = int(run.cache.length.max())
    c = run.cache
    exact = [c.k, c.v, c.m[:, :L], c.pos[:, :L], c.length, run.lse, run.s[:, :L + 1]]
    if c.votes is not None:
        exact.append(c.votes[:, :L])
    if run.mom is not None:
        exact += [run.mom.n, run.mom.sk, run.mom.sv, run.mom.S]
    return [bits(x) for x in exact], bits(run.out).astype(np.float64)


@pytest.mark.parametrize("path", list(CASES))
def test_resume_from_checkpoint_matches_straight_run(path):
    wl, merge = CASES[path]
    T = wl.steps
    straight = DeviceRun(wl, max_len=_run_max_len(wl, path))
    for step in range(1, T + 1):
        _step(straight, wl, path, step, merge)
    ref_exact, ref_out = _state(straight)
    del straight

    first = DeviceRun(wl, max_len=_run_max_len(wl, path))
    for step in range(1, T // 2 + 1):
        _step(first, wl, path, step, merge)
    torch.cuda.synchronize()
    blob = _save(first)
    del first
    resumed = _restore(wl, path, blob)
    for step in range(T // 2 + 1, T + 1):
        _step(resumed, wl, path, step, merge)
    got_exact, got_out = _state(resumed)

    assert resumed.t == wl.context + T
    for i, (a, b) in enumerate(zip(ref_exact, got_exact)):
        assert a.shape == b.shape and np.array_equal(a, b), f"state tensor {i} differs after resume"
    assert np.all(np.abs(ref_out - got_out) <= 1e-6 * np.abs(ref_out).max(axis=-1, keepdims=True))

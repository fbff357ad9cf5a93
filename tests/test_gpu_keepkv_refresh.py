"""GPU parity of KeepKV's periodic refresh (kvc_keepkv_refresh) against oracle.refresh.

The cache starts in an unrelated compressed state (other rows, votes, utilities, positions and
lengths); the full KV of every head (prompt and decode tokens so far) sits in pinned host memory.
After the call the oracle replays each scope's merge sequence on the reloaded bytes: at every
round the GPU's pair must have the largest cosine of the current entries or lie within 1e-6
(relative) of it. Compared after the refresh, by position:
  * the live positions and the live length (the budget), exactly; the workspace status;
  * votes exactly; rows: untouched rows bit-exact (the host bytes), merged rows within one unit in
    the last place of bf16; utilities (the restarted EMA window sums, added over merges) within
    1e-5 relative (float32 weights on the device);
  * a second refresh from the same host store gives the same cache (nothing of the first refresh
    or of the prior state leaks into it).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import bits
from oracle.keepkv_prefill import best_pair, cosine_matrix

pytestmark = pytest.mark.gpu

D = 128
SCALE = float(np.float32(1.0 / np.sqrt(D)))
BAND = 1e-6


def _setup(S, cap, n, n_win, G, seed):
    # prior state: unrelated rows, votes, utilities, positions and lengths
    K0, V0 = synth.kv_rows(S, cap, D, "bf16", seed + 100, "cuda", synth.key_scales(S, D, seed + 100, "cuda"))
    gen = np.random.default_rng(seed)
    cache = kvc.Cache(k=K0.view(S, 1, cap, D).contiguous(), v=V0.view(S, 1, cap, D).contiguous(),
                      pos=torch.from_numpy(gen.permutation(10 * cap)[:cap].astype(np.int32)).repeat(S, 1).cuda(),
                      m=torch.from_numpy(gen.random((S, cap)).astype(np.float32)).cuda(),
                      length=torch.from_numpy(gen.integers(1, cap, size=S).astype(np.int32)).cuda(),
                      votes=torch.from_numpy(gen.integers(1, 5, size=(S, cap)).astype(np.int32)).cuda())
    # the full KV in pinned host memory, positions 0 .. n-1
    Kf, Vf = synth.kv_rows(S, n, D, "bf16", seed, "cpu", synth.key_scales(S, D, seed, "cpu"))
    hk = torch.empty((S, n, D), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((S, n, D), dtype=torch.bfloat16, pin_memory=True)
    hp = torch.empty((S, n), dtype=torch.int32, pin_memory=True)
    hk.copy_(Kf.view(S, n, D))
    hv.copy_(Vf.view(S, n, D))
    hp.copy_(torch.arange(n, dtype=torch.int32).repeat(S, 1))
    # the last n_win steps' queries; the current step's is the last row
    q_win = torch.stack([synth.step_query(j, S, G, D, "bf16", seed, "cuda") for j in range(n_win)], dim=2).contiguous()
    q_ref = q_win[:, :, -1, :].contiguous()
    return cache, hk, hv, hp, q_win, q_ref


def _refresh(cache, hk, hv, hp, n, q_win, n_win, q_ref, G, alpha, budget, protect_from):
    S, cap = cache.n_scopes, cache.capacity
    pairs = torch.full((S, cap, 2), -1, dtype=torch.int32, device="cuda")
    n_merged = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_keepkv_refresh_workspace_size(cache, G, n_win, n))
    kvc.kvc_keepkv_refresh(cache, hk, hv, hp, n, q_win, n_win, kvc.merge_desc(q_ref, G, SCALE), alpha, budget,
                           protect_from, pairs, n_merged, ws=ws)
    torch.cuda.synchronize()
    return pairs.cpu().numpy(), n_merged.cpu().numpy(), kvc.kvc_workspace_status(ws)


def _state(cache):
    L = cache.length.cpu().numpy()
    return {"len": L, "k": bits(cache.k[:, 0]), "v": bits(cache.v[:, 0]), "votes": cache.votes.cpu().numpy(),
            "pos": cache.pos.cpu().numpy(), "m": cache.m.cpu().numpy().astype(np.float64)}


@pytest.mark.parametrize("S,n,n_win,G,budget,R", [(4, 700, 16, 4, 70, 8), (3, 1100, 32, 8, 110, 32),
                                                  (2, 400, 8, 1, 41, 4)])
def test_refresh_matches_oracle(S, n, n_win, G, budget, R):
    cap, alpha, seed = n + 300, 0.9, 7 + n
    cache, hk, hv, hp, q_win, q_ref = _setup(S, cap, n, n_win, G, seed)
    protect_from = n - R
    pr, nm, status = _refresh(cache, hk, hv, hp, n, q_win, n_win, q_ref, G, alpha, budget, protect_from)
    assert status == 0
    post = _state(cache)
    assert np.all(post["len"] == budget)
    Kb, Vb = bits(hk).reshape(S, n, D), bits(hv).reshape(S, n, D)
    qw, qr = oracle.to_f64(bits(q_win), "bf16"), oracle.to_f64(bits(q_ref), "bf16")
    pos = np.arange(n)
    flips = 0
    for sc in range(S):
        K = oracle.to_f64(Kb[sc], "bf16")
        V = oracle.to_f64(Vb[sc], "bf16")

        def follow(step, Kc, cand):
            nonlocal flips
            if step >= nm[sc]:
                assert best_pair(Kc, pos, cand) is None, f"scope {sc}: oracle wants merge {step}, GPU did {nm[sc]}"
                return None
            s_, g_ = int(pr[sc, step, 0]), int(pr[sc, step, 1])
            assert cand[s_] and cand[g_], f"scope {sc} step {step}: GPU pair ({s_}, {g_}) not mergeable"
            bi, bj, bc = best_pair(Kc, pos, cand)
            if {s_, g_} != {bi, bj}:
                cg = cosine_matrix(Kc[[s_, g_]])[0, 1]
                assert cg >= bc - BAND * abs(bc), f"scope {sc} step {step}: cos {cg!r} vs best {bc!r}"
                flips += 1
            return s_, g_

        res = oracle.refresh(K, V, pos, qw[sc], qr[sc], SCALE, alpha, budget, protect_from, row_dtype="bf16",
                             choose=follow)
        assert len(res["pairs"]) == nm[sc]
        live = np.flatnonzero(res["live"])
        L = int(post["len"][sc])
        gpos = post["pos"][sc, :L]
        assert sorted(gpos.tolist()) == live.tolist(), f"scope {sc}: live positions"
        merged = {s_ for s_, _ in res["pairs"]}
        for slot, p in enumerate(gpos.tolist()):
            assert post["votes"][sc, slot] == res["votes"][p]
            if p in merged:
                for got, ref in ((post["k"][sc, slot], res["K"][p]), (post["v"][sc, slot], res["V"][p])):
                    g = oracle.to_f64(got, "bf16")
                    assert np.all(np.abs(g - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), f"scope {sc} pos {p}: rows"
            else:
                assert np.array_equal(post["k"][sc, slot], Kb[sc, p]) and np.array_equal(post["v"][sc, slot], Vb[sc, p])
            assert abs(post["m"][sc, slot] - res["m"][p]) <= 1e-5 * abs(res["m"][p]) + 1e-12, f"scope {sc} pos {p}: m"
    print(f"refresh S={S} n={n} G={G}: merges {list(nm)}, near-tie picks {flips}", flush=True)

    # a second refresh from the same host store gives the same cache
    first = post
    pr2, nm2, status2 = _refresh(cache, hk, hv, hp, n, q_win, n_win, q_ref, G, alpha, budget, protect_from)
    assert status2 == 0 and np.array_equal(nm2, nm) and np.array_equal(pr2, pr)
    second = _state(cache)
    for key in ("len", "k", "v", "votes", "pos", "m"):
        a, b = first[key], second[key]
        if key in ("k", "v"):
            a, b = a[:, :budget], b[:, :budget]
        elif key != "len":
            a, b = a[:, :budget], b[:, :budget]
        assert np.array_equal(a, b), key

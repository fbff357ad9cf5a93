"""GPU parity of MomentKV moment-informed eviction (kvc_moment_evict) with the fp64 oracle (MI355X).

Each case hands the oracle host copies of exactly the bytes the GPU consumed (K, V, positions,
weights, moment sums) and compares:
  * evictions: in every round the GPU's pick is the oracle's lowest score, or lies within 1e-6
    (relative) of it; the oracle then follows the GPU's pick into the next round;
  * first-round scores: 1e-6 relative (the GPU rounds its float64 score to fp32);
  * moment sums after the fold: n exact; s_k, s_v, S within 1e-6 of the summed magnitudes of the
    input sums and the folded terms (one fp32 rounding per fold);
  * flags: 1 exactly on the evicted slots below len, 0 on the other live slots, untouched above;
  * the eviction order and the per-scope counts.
Shapes span ragged tiles and chunks (lengths 1 past a 64-token boundary), empty and under-budget
scopes, empty sums (n_e = 0), one evicted token, and sums scaled so that the key-dependent part of
the moment model is as large as the values.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import bits
from oracle.moment_evict import moment_informed_evict

pytestmark = pytest.mark.gpu

D = 128
SCALE = float(np.float32(1.0 / np.sqrt(D)))
BAND = 1e-6


def _make(lens, cap, dtype, n_e, seed, s_scale=1.0, device="cuda"):
    S = len(lens)
    K, V = synth.kv_rows(S, cap, D, dtype, seed, device)
    pos = synth.initial_positions(S, cap, 8 * cap, seed, device)
    length = torch.tensor(lens, dtype=torch.int32, device=device)
    cache = kvc.Cache(k=K.view(S, 1, cap, D).contiguous(), v=V.view(S, 1, cap, D).contiguous(), pos=pos,
                      m=torch.zeros((S, cap), device=device), length=length)
    ms = synth.moment_sums(S, D, n_e, seed, device, s_scale=s_scale)
    mom = kvc.Moments(ms["n"].view(S, 1).contiguous(), ms["sk"].view(S, 1, D).contiguous(),
                      ms["sv"].view(S, 1, D).contiguous(), ms["S"].view(S, 1, D, D).contiguous())
    w = synth.token_weights(S, cap, seed, device).double()
    live = torch.arange(cap, device=device)[None, :] < length[:, None].long()
    w = torch.where(live, w, torch.zeros_like(w))
    alpha = (w / w.sum(dim=1, keepdim=True).clamp_min(1e-300)).float().contiguous()
    return cache, mom, alpha


def _host(cache, mom, alpha, dtype):
    h = {"len": cache.length.cpu().numpy(), "k": bits(cache.k[:, 0]), "v": bits(cache.v[:, 0]),
         "pos": cache.pos.cpu().numpy(), "alpha": alpha.cpu().numpy(), "n": mom.n[:, 0].cpu().numpy(),
         "sk": mom.sk[:, 0].cpu().numpy(), "sv": mom.sv[:, 0].cpu().numpy(), "S": mom.S[:, 0].cpu().numpy()}
    h["dtype"] = dtype
    return h


def _oracle_scope(h, sc, budget, gpu_order):
    """Run the oracle on scope sc following the GPU's picks; check each pick is the lowest or within the band."""
    L = int(h["len"][sc])
    K = oracle.to_f64(h["k"][sc, :L], h["dtype"])
    V = oracle.to_f64(h["v"][sc, :L], h["dtype"])
    mom_in = {"n": int(h["n"][sc]), "sk": h["sk"][sc].astype(np.float64), "sv": h["sv"][sc].astype(np.float64),
              "S": h["S"][sc].astype(np.float64)}
    flips = [0]

    def follow(step, scores, live):
        e = int(gpu_order[step])
        assert 0 <= e < L and live[e], f"scope {sc} round {step}: GPU evicted slot {e} (not live)"
        best = float(scores[live].min())
        if scores[e] != best:
            assert scores[e] <= best * (1.0 + BAND), \
                f"scope {sc} round {step}: GPU pick {e} score {scores[e]!r} vs lowest {best!r}"
            flips[0] += 1
        return e

    order, mom_out, first, _ = moment_informed_evict(K, V, h["alpha"][sc, :L].astype(np.float64),
                                                     h["pos"][sc, :L], mom_in, budget, SCALE, choose=follow)
    return order, mom_out, first, mom_in, flips[0]


def _run(cache, mom, alpha, budget, max_len, preset=7):
    S, C = cache.n_scopes, cache.capacity
    evict = torch.full((S, C), preset, dtype=torch.uint8, device="cuda")
    order = torch.full((S, C), -1, dtype=torch.int32, device="cuda")
    score = torch.full((S, C), -1.0, device="cuda")
    n_ev = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_moment_evict_workspace_size(cache))
    kvc.kvc_moment_evict(cache, mom, alpha, SCALE, budget, evict, order, score, n_ev, max_len=max_len, ws=ws)
    torch.cuda.synchronize()
    return evict.cpu().numpy(), order.cpu().numpy(), score.cpu().numpy(), n_ev.cpu().numpy(), ws


def _check(h, mom, budget, evict, order, score, n_ev, preset=7):
    S = len(h["len"])
    n_after = mom.n[:, 0].cpu().numpy()
    sk_after, sv_after, S_after = (mom.sk[:, 0].cpu().numpy(), mom.sv[:, 0].cpu().numpy(),
                                   mom.S[:, 0].cpu().numpy())
    total_flips = 0
    for sc in range(S):
        L = int(h["len"][sc])
        k = max(0, L - budget)
        assert n_ev[sc] == k, f"scope {sc}: n_evict {n_ev[sc]} != {k}"
        gpu_order = order[sc, :k]
        ref_order, mom_ref, first, mom_in, flips = _oracle_scope(h, sc, budget, gpu_order)
        total_flips += flips
        assert len(ref_order) == k
        # flags
        want = np.zeros(L, dtype=np.uint8)
        want[gpu_order] = 1
        assert np.array_equal(evict[sc, :L], want), f"scope {sc}: flags"
        assert np.all(evict[sc, L:] == preset), f"scope {sc}: flags above len were written"
        assert len(set(gpu_order.tolist())) == k
        # first-round scores
        if L > 0:
            np.testing.assert_allclose(score[sc, :L], first, rtol=BAND, atol=1e-30,
                                       err_msg=f"scope {sc}: first-round scores")
        # sums
        assert n_after[sc] == mom_ref["n"], f"scope {sc}: n"
        # one fp32 rounding per fold: bound by the summed magnitudes of the folded terms
        Ke = oracle.to_f64(h["k"][sc, gpu_order], h["dtype"])
        Ve = oracle.to_f64(h["v"][sc, gpu_order], h["dtype"])
        mag = {"sk": np.abs(Ke).sum(axis=0), "sv": np.abs(Ve).sum(axis=0), "S": np.abs(Ve).T @ np.abs(Ke)}
        for name, got in (("sk", sk_after[sc]), ("sv", sv_after[sc]), ("S", S_after[sc])):
            ref = mom_ref[name]
            tol = 1e-6 * (np.abs(mom_in[name]) + mag[name]) + 1e-30
            err = np.abs(got.astype(np.float64) - ref)
            assert np.all(err <= tol), f"scope {sc}: {name} err {(err / (tol + 1e-30)).max()}x tol"
    return total_flips


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("s_scale", [1.0, 40.0])
def test_single_round(dtype, s_scale):
    budget = 128
    lens = [0, 100, 128, 129, 129, 129, 129, 129, 65, 129]
    n_e = [0, 5, 7, 0, 1, 2, 500, 40000, 3, 30000]
    cache, mom, alpha = _make(lens, 300, dtype, n_e, seed=11 + int(s_scale), s_scale=s_scale)
    h = _host(cache, mom, alpha, dtype)
    evict, order, score, n_ev, ws = _run(cache, mom, alpha, budget, budget + 1)
    flips = _check(h, mom, budget, evict, order, score, n_ev)
    assert kvc.kvc_workspace_status(ws) == 0
    print(f"single round {dtype} s_scale={s_scale}: near-tie flips {flips}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_several_rounds_rescore_after_each_fold(dtype):
    budget = 150
    lens = [150, 151, 158, 166, 0, 166]
    n_e = [0, 3, 0, 1000, 0, 1]
    cache, mom, alpha = _make(lens, 200, dtype, n_e, seed=23, s_scale=20.0)
    h = _host(cache, mom, alpha, dtype)
    evict, order, score, n_ev, ws = _run(cache, mom, alpha, budget, max(lens))
    flips = _check(h, mom, budget, evict, order, score, n_ev)
    assert kvc.kvc_workspace_status(ws) == 0
    print(f"several rounds {dtype}: near-tie flips {flips}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_one_chunk_per_scope_picks_inside_the_score_kernel(dtype):
    """More scopes than CUs: each scope is one chunk, and the score kernel's workgroup
    picks and folds itself (no second kernel); ragged lengths, up to 4 rounds, empty scopes."""
    budget, S = 150, 260
    rng = np.random.default_rng(3)
    lens = [int(x) for x in rng.integers(0, budget + 5, size=S)]
    lens[:6] = [0, budget, budget + 1, budget + 4, 1, budget + 2]
    n_e = [int(x) for x in rng.integers(0, 3000, size=S)]
    cache, mom, alpha = _make(lens, budget + 4, dtype, n_e, seed=31, s_scale=15.0)
    h = _host(cache, mom, alpha, dtype)
    evict, order, score, n_ev, ws = _run(cache, mom, alpha, budget, budget + 4)
    flips = _check(h, mom, budget, evict, order, score, n_ev)
    assert kvc.kvc_workspace_status(ws) == 0
    print(f"one chunk per scope {dtype}: near-tie flips {flips}", flush=True)


def test_too_few_rounds_sets_the_status():
    """max_len below a scope's live length: that scope evicts as many as the rounds allow."""
    budget = 64
    cache, mom, alpha = _make([65, 67, 64], 80, "bf16", [10, 10, 10], seed=5)
    evict, order, score, n_ev, ws = _run(cache, mom, alpha, budget, budget + 1)
    assert list(n_ev) == [1, 1, 0]
    assert int(evict[1, :67].sum()) == 1 and int(evict[0, :65].sum()) == 1
    assert kvc.kvc_workspace_status(ws) == -4          # KVC_ERR_CAPACITY


def test_full_size_steady_step():
    """32 layers x 8 KV heads at budget 1024, 1025 live tokens each, one eviction per head
    (the launch configuration the benchmark times); every head is checked."""
    wl = synth.WORKLOADS["m1_momentkv_llama8b_32layers_b1024"]
    L = wl.budget + 1
    S = wl.n_scopes
    cache, mom, alpha = _make([L] * S, L, wl.dtype, wl.context - wl.budget, seed=wl.seed)
    h = _host(cache, mom, alpha, wl.dtype)
    evict, order, score, n_ev, ws = _run(cache, mom, alpha, wl.budget, L)
    flips = _check(h, mom, wl.budget, evict, order, score, n_ev)
    assert kvc.kvc_workspace_status(ws) == 0
    print(f"full size: {S} heads, near-tie flips {flips}", flush=True)


@pytest.mark.parametrize("name,budget,n_kv,steps", [("c1_head_f32_4k", 128, 1, 6),
                                                     ("c2_llama8b_layer_32k", 1024, 8, 3)])
def test_composed_decode_steps(name, budget, n_kv, steps):
    """kvc_decode_attn_score (append, attention, head-averaged weights) -> kvc_moment_evict
    (alpha = those weights) -> kvc_compact, step by step; the oracle attends, scores and evicts
    from the same pre-state with its own weights."""
    wl = synth.WORKLOADS[name].scaled(budget=budget, context=budget, n_kv=n_kv, steps=steps)
    t = synth.cache_tensors(wl, "cuda", capacity=budget + 1, initial_len=budget)
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"])
    S, C, G = wl.n_scopes, budget + 1, wl.G
    ms = synth.moment_sums(S, D, 4 * budget, wl.seed, "cuda", s_scale=10.0)
    mom = kvc.Moments(ms["n"].view(S, 1).contiguous(), ms["sk"].view(S, 1, D).contiguous(),
                      ms["sv"].view(S, 1, D).contiguous(), ms["S"].view(S, 1, D, D).contiguous())
    out = torch.empty((S, 1, G, D), device="cuda")
    lse = torch.empty((S, 1, G), device="cuda")
    s = torch.empty((S, C), device="cuda")
    evict = torch.zeros((S, C), dtype=torch.uint8, device="cuda")
    order = torch.full((S, C), -1, dtype=torch.int32, device="cuda")
    ws_a = kvc.workspace(kvc.kvc_decode_workspace_size(cache, G, C))
    ws_m = kvc.workspace(kvc.kvc_moment_evict_workspace_size(cache))
    ws_c = kvc.workspace(kvc.kvc_compact_workspace_size(cache))
    flips = 0
    for step in range(1, steps + 1):
        q, kn, vn = synth.step_inputs(wl, step, t["scales"], "cuda")
        pre = {"k": bits(cache.k[:, 0]), "v": bits(cache.v[:, 0]), "pos": cache.pos.cpu().numpy(),
               "len": cache.length.cpu().numpy(), "n": mom.n[:, 0].cpu().numpy(),
               "sk": mom.sk[:, 0].cpu().numpy(), "sv": mom.sv[:, 0].cpu().numpy(), "S": mom.S[:, 0].cpu().numpy()}
        qh, knh, vnh = bits(q), bits(kn), bits(vn)
        tpos = wl.context + step - 1
        kvc.kvc_decode_attn_score(cache, kn, vn, tpos, q, G, SCALE, out, lse, s, C, ws_a)
        kvc.kvc_moment_evict(cache, mom, s, SCALE, budget, evict, order, max_len=C, ws=ws_m)
        ev = evict.cpu().numpy()
        ordh = order.cpu().numpy()
        kvc.kvc_compact(cache, evict, None, ws_c)
        torch.cuda.synchronize()
        for sc in range(S):
            L0 = int(pre["len"][sc])
            K = np.vstack([oracle.to_f64(pre["k"][sc, :L0], wl.dtype), oracle.to_f64(knh[sc, 0][None], wl.dtype)])
            V = np.vstack([oracle.to_f64(pre["v"][sc, :L0], wl.dtype), oracle.to_f64(vnh[sc, 0][None], wl.dtype)])
            pos = np.append(pre["pos"][sc, :L0], tpos)
            _, a, _, _ = oracle.attend_unit(oracle.to_f64(qh[sc, 0], wl.dtype), K, V, None, SCALE)
            alpha = oracle.scope_score([a])
            mom_in = {"n": int(pre["n"][sc]), "sk": pre["sk"][sc].astype(np.float64),
                      "sv": pre["sv"][sc].astype(np.float64), "S": pre["S"][sc].astype(np.float64)}
            e_gpu = int(ordh[sc, 0])

            def follow(i, scores, live):
                nonlocal flips
                best = float(scores[live].min())
                if scores[e_gpu] != best:
                    assert scores[e_gpu] <= best * (1.0 + BAND), (sc, step, e_gpu, scores[e_gpu], best)
                    flips += 1
                return e_gpu

            ref_order, mom_ref, _, _ = moment_informed_evict(K, V, alpha, pos, mom_in, budget, SCALE, choose=follow)
            assert list(ref_order) == [e_gpu] and ev[sc, :L0 + 1].sum() == 1 and ev[sc, e_gpu] == 1
            # the cache after compaction holds the other tokens, rows bit-exact
            L1 = int(cache.length[sc])
            assert L1 == budget
            keep = np.ones(L0 + 1, dtype=bool)
            keep[e_gpu] = False
            post_pos = cache.pos[sc, :L1].cpu().numpy()
            assert sorted(post_pos.tolist()) == sorted(pos[keep].tolist())
            post_k = oracle.to_f64(bits(cache.k[sc, 0, :L1]), wl.dtype)
            by_pos = {int(p): i for i, p in enumerate(pos)}
            idx = np.array([by_pos[int(p)] for p in post_pos])
            assert np.array_equal(post_k, K[idx])
            assert int(mom.n[sc, 0]) == mom_ref["n"]
            err = np.abs(mom.S[sc, 0].cpu().numpy().astype(np.float64) - mom_ref["S"])
            assert np.all(err <= 1e-6 * (np.abs(mom_in["S"]) + np.abs(np.outer(V[e_gpu], K[e_gpu]))) + 1e-30)
    print(f"composed {name}: {steps} steps x {S} heads, near-tie flips {flips}", flush=True)

"""GPU parity of KeepKV prefill compression by greedy all-pairs ZIP merging (kvc_keepkv_prefill_merge).

The oracle replays each scope's merge sequence on the very bytes the GPU consumed: at every
round it checks that the GPU's pair has the largest cosine of the current entries, or lies
within 1e-6 (relative) of it, then follows that pair. Compared afterwards:
  * the number of merges and the removed slots (flags), exactly;
  * votes exactly; the rows of every live slot: untouched rows bit-exact, merged rows within one
    unit in the last place of the cache dtype (the merge's float64 arithmetic runs in another
    order); utilities within 1e-6 relative (fp32 sums);
  * after kvc_compact, every scope holds the oracle's live positions.
Shapes: ragged lengths per scope, a scope already within budget, protected recent positions,
G = 1, 4, 8, bf16 and fp32 caches, and a scope that cannot reach its budget (status).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import bits
from oracle.keepkv_prefill import best_pair, cosine_matrix, prefill_merge

pytestmark = pytest.mark.gpu

D = 128
SCALE = float(np.float32(1.0 / np.sqrt(D)))
BAND = 1e-6


def _make(lens, cap, dtype, G, seed):
    S = len(lens)
    scales = synth.key_scales(S, D, seed, "cuda")
    K, V = synth.kv_rows(S, cap, D, dtype, seed, "cuda", scales)
    pos = torch.arange(cap, dtype=torch.int32, device="cuda").repeat(S, 1).contiguous()
    m = synth.token_weights(S, cap, seed, "cuda").contiguous()
    cache = kvc.Cache(k=K.view(S, 1, cap, D).contiguous(), v=V.view(S, 1, cap, D).contiguous(), pos=pos, m=m,
                      length=torch.tensor(lens, dtype=torch.int32, device="cuda"),
                      votes=torch.ones((S, cap), dtype=torch.int32, device="cuda"))
    q = synth.step_query(1, S, G, D, dtype, seed, "cuda").contiguous()
    return cache, q


def _host(cache):
    return {"k": bits(cache.k[:, 0]), "v": bits(cache.v[:, 0]), "votes": cache.votes.cpu().numpy(),
            "pos": cache.pos.cpu().numpy(), "m": cache.m.cpu().numpy().astype(np.float64),
            "len": cache.length.cpu().numpy()}


def _ulp_close(got, ref, dtype):
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -23
    return np.all(np.abs(got - ref) <= rel * np.abs(ref) + 1e-30)


def _run_and_check(lens, cap, budget, protect_from, dtype, G, seed, expect_status=0):
    cache, q = _make(lens, cap, dtype, G, seed)
    S = len(lens)
    pre = _host(cache)
    qh = oracle.to_f64(bits(q), dtype)
    evict = torch.full((S, cap), 7, dtype=torch.uint8, device="cuda")
    pairs = torch.full((S, cap, 2), -1, dtype=torch.int32, device="cuda")
    n_merged = torch.full((S,), -1, dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_keepkv_prefill_workspace_size(cache))
    merge = kvc.merge_desc(q, G, SCALE)
    kvc.kvc_keepkv_prefill_merge(cache, merge, budget, protect_from, evict, pairs, n_merged, ws=ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_status(ws) == expect_status
    post = _host(cache)
    ev, pr, nm = evict.cpu().numpy(), pairs.cpu().numpy(), n_merged.cpu().numpy()
    flips = 0
    ref = []
    for sc in range(S):
        L = int(pre["len"][sc])
        K = oracle.to_f64(pre["k"][sc, :L], dtype)
        V = oracle.to_f64(pre["v"][sc, :L], dtype)
        pos = pre["pos"][sc, :L]

        def follow(step, Kc, cand):
            nonlocal flips
            if step >= nm[sc]:     # the GPU stopped: so must the oracle (no mergeable pair left)
                assert best_pair(Kc, pos, cand) is None, f"scope {sc}: oracle wants merge {step}, GPU did {nm[sc]}"
                return None
            s_, g_ = int(pr[sc, step, 0]), int(pr[sc, step, 1])
            assert cand[s_] and cand[g_], f"scope {sc} step {step}: GPU pair ({s_}, {g_}) not mergeable"
            bi, bj, bc = best_pair(Kc, pos, cand)
            cg = cosine_matrix(Kc[[s_, g_]])[0, 1]
            if {s_, g_} != {bi, bj}:
                assert cg >= bc - BAND * abs(bc), f"scope {sc} step {step}: cos {cg!r} vs best {bc!r}"
                flips += 1
            return s_, g_

        res = prefill_merge(K, V, pre["votes"][sc, :L], pos, pre["m"][sc, :L], qh[sc], SCALE, budget,
                            protect_from, row_dtype=dtype, choose=follow)
        assert len(res["pairs"]) == nm[sc], f"scope {sc}: {len(res['pairs'])} merges vs GPU {nm[sc]}"
        gone = np.zeros(L, dtype=np.uint8)
        for s_, g_ in res["pairs"]:
            gone[g_] = 1
        assert np.array_equal(ev[sc, :L], gone) and np.all(ev[sc, L:] == 7), f"scope {sc}: flags"
        live = res["live"]
        assert np.array_equal(post["votes"][sc, :L][live], res["votes"][live])
        Kg = oracle.to_f64(post["k"][sc, :L], dtype)[live]
        Vg = oracle.to_f64(post["v"][sc, :L], dtype)[live]
        assert _ulp_close(Kg, res["K"][live], dtype) and _ulp_close(Vg, res["V"][live], dtype), f"scope {sc}: rows"
        untouched = live.copy()
        for s_, _ in res["pairs"]:
            untouched[s_] = False
        assert np.array_equal(post["k"][sc, :L][untouched], pre["k"][sc, :L][untouched])
        np.testing.assert_allclose(post["m"][sc, :L][live], res["m"][live], rtol=1e-6, atol=1e-12)
        ref.append(set(pos[live].tolist()))
    # compaction removes the flagged slots
    ws_c = kvc.workspace(kvc.kvc_compact_workspace_size(cache))
    kvc.kvc_compact(cache, evict, None, ws_c)
    torch.cuda.synchronize()
    lens_after = cache.length.cpu().numpy()
    pos_after = cache.pos.cpu().numpy()
    for sc in range(S):
        assert set(pos_after[sc, :lens_after[sc]].tolist()) == ref[sc]
    print(f"prefill merge S={S} {dtype} G={G}: merges {list(nm)}, near-tie picks {flips}", flush=True)


@pytest.mark.parametrize("dtype,G", [("bf16", 4), ("f32", 1), ("bf16", 8)])
def test_prefill_merge_matches_oracle(dtype, G):
    lens = [200, 150, 90, 30]
    _run_and_check(lens, 200, budget=40, protect_from=192, dtype=dtype, G=G, seed=41 + G)


def test_prefill_merge_longer_prompt():
    _run_and_check([700, 523], 700, budget=70, protect_from=690, dtype="bf16", G=4, seed=5)


def test_prefill_merge_stops_when_the_budget_cannot_be_reached():
    # positions >= 20 are protected: 60 - 20 = 40 entries never merge, so a budget of 30 is out of reach
    _run_and_check([60, 25], 60, budget=30, protect_from=20, dtype="bf16", G=4, seed=9, expect_status=-4)


def test_prefill_merge_full_size_sampled():
    """The benchmarked configuration: 256 KV heads x 4096-token prompts -> 409 entries, the last
    32 positions protected, G = 4. Every head: exactly 3687 merges, votes conserved (sum 4096),
    protected rows untouched, removed slots flagged once. Two sampled heads: the first 24 merges
    replayed in the oracle (each GPU pair the largest cosine, or within 1e-6 of it)."""
    wl = synth.WORKLOADS["k1_keepkv_prefill_llama8b_4k"]
    S, L0, B = wl.n_scopes, wl.context, wl.budget
    protect_from = L0 - 32
    t = synth.cache_tensors(wl, "cuda")
    votes = torch.ones((S, t["k"].shape[2]), dtype=torch.int32, device="cuda")
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"], votes=votes)
    cap = cache.capacity
    q = synth.step_query(0, S, wl.G, D, wl.dtype, wl.seed, "cuda").contiguous()
    pre_k = bits(cache.k[:, 0])
    pre_pos = cache.pos.cpu().numpy()
    evict = torch.zeros((S, cap), dtype=torch.uint8, device="cuda")
    pairs = torch.full((S, cap, 2), -1, dtype=torch.int32, device="cuda")
    n_merged = torch.zeros((S,), dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_keepkv_prefill_workspace_size(cache))
    kvc.kvc_keepkv_prefill_merge(cache, kvc.merge_desc(q, wl.G, SCALE), B, protect_from, evict, pairs, n_merged,
                                 ws=ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_status(ws) == 0
    nm, ev, pr = n_merged.cpu().numpy(), evict.cpu().numpy(), pairs.cpu().numpy()
    vt = cache.votes.cpu().numpy()
    post_k = bits(cache.k[:, 0])
    assert np.all(nm == L0 - B)
    for sc in range(S):
        gone = ev[sc, :L0].astype(bool)
        assert gone.sum() == L0 - B
        assert vt[sc, :L0][~gone].sum() == L0
        prot = pre_pos[sc, :L0] >= protect_from
        assert not np.any(gone & prot)
        assert np.array_equal(post_k[sc, :L0][prot], pre_k[sc, :L0][prot])
        g = pr[sc, :L0 - B, 1]
        assert np.array_equal(np.sort(g), np.flatnonzero(gone))
    n_rep = 24
    for sc in (0, 201):
        K = oracle.to_f64(pre_k[sc, :L0], "bf16")
        pos = pre_pos[sc, :L0]

        def follow(step, Kc, cand):
            s_, g_ = int(pr[sc, step, 0]), int(pr[sc, step, 1])
            assert cand[s_] and cand[g_]
            bi, bj, bc = best_pair(Kc, pos, cand)
            cg = cosine_matrix(Kc[[s_, g_]])[0, 1]
            assert {s_, g_} == {bi, bj} or cg >= bc - BAND * abs(bc), (sc, step, cg, bc)
            return s_, g_

        qh = oracle.to_f64(bits(q[sc]), "bf16")
        res = prefill_merge(K, np.zeros_like(K), np.ones(L0, dtype=np.int64), pos, np.zeros(L0), qh, SCALE,
                            L0 - n_rep, protect_from, row_dtype="bf16", choose=follow)
        assert len(res["pairs"]) == n_rep
        print(f"full-size prefill merge: head {sc}, first {n_rep} merges follow the oracle", flush=True)


def test_prefill_merge_many_exact_ties():
    """Heads whose keys take two values (1300 copies of one, 236 of the other): merging two copies
    gives the same key, so every copy ties the merged key at its list's last entry and a merge
    pass finds more rows whose list may change than it queues (they are handled in the pass).
    Checked: exactly L - B merges per head, votes conserved, protected rows untouched, removed
    slots flagged once; the first 16 merges of two heads replayed in the oracle (each GPU pair the
    largest cosine, or within 1e-6 of it)."""
    S, L0, B = 4, 1536, 600
    protect_from = L0 - 32
    gen = torch.Generator().manual_seed(77)
    rows = torch.randn((S, 2, D), generator=gen).to(torch.bfloat16)
    cls = torch.zeros((S, L0), dtype=torch.long)
    for sc in range(S):
        cls[sc, torch.randperm(L0, generator=gen)[:236]] = 1
    K = torch.stack([rows[sc][cls[sc]] for sc in range(S)]).contiguous()
    V = torch.randn((S, L0, D), generator=gen).to(torch.bfloat16)
    cache = kvc.Cache(k=K.view(S, 1, L0, D).cuda(), v=V.view(S, 1, L0, D).cuda(),
                      pos=torch.arange(L0, dtype=torch.int32).repeat(S, 1).cuda(),
                      m=torch.zeros((S, L0), dtype=torch.float32).cuda(),
                      length=torch.full((S,), L0, dtype=torch.int32).cuda(),
                      votes=torch.ones((S, L0), dtype=torch.int32).cuda())
    q = torch.randn((S, 4, D), generator=gen).to(torch.bfloat16).cuda().contiguous()
    pre_k = bits(cache.k[:, 0])
    evict = torch.zeros((S, L0), dtype=torch.uint8, device="cuda")
    pairs = torch.full((S, L0, 2), -1, dtype=torch.int32, device="cuda")
    n_merged = torch.zeros((S,), dtype=torch.int32, device="cuda")
    ws = kvc.workspace(kvc.kvc_keepkv_prefill_workspace_size(cache))
    kvc.kvc_keepkv_prefill_merge(cache, kvc.merge_desc(q, 4, SCALE), B, protect_from, evict, pairs, n_merged, ws=ws)
    torch.cuda.synchronize()
    assert kvc.kvc_workspace_status(ws) == 0
    nm, ev, pr = n_merged.cpu().numpy(), evict.cpu().numpy(), pairs.cpu().numpy()
    vt = cache.votes.cpu().numpy()
    post_k = bits(cache.k[:, 0])
    assert np.all(nm == L0 - B)
    for sc in range(S):
        gone = ev[sc].astype(bool)
        assert gone.sum() == L0 - B and vt[sc][~gone].sum() == L0
        assert not np.any(gone[protect_from:])
        assert np.array_equal(post_k[sc, protect_from:], pre_k[sc, protect_from:])
        assert np.array_equal(np.sort(pr[sc, :L0 - B, 1]), np.flatnonzero(gone))
    n_rep = 16
    pos = np.arange(L0)
    for sc in (0, 3):
        Kh = oracle.to_f64(pre_k[sc], "bf16")

        def follow(step, Kc, cand):
            s_, g_ = int(pr[sc, step, 0]), int(pr[sc, step, 1])
            assert cand[s_] and cand[g_]
            bi, bj, bc = best_pair(Kc, pos, cand)
            cg = cosine_matrix(Kc[[s_, g_]])[0, 1]
            assert {s_, g_} == {bi, bj} or cg >= bc - BAND * abs(bc), (sc, step, cg, bc)
            return s_, g_

        qh = oracle.to_f64(bits(q[sc]), "bf16")
        res = prefill_merge(Kh, np.zeros_like(Kh), np.ones(L0, dtype=np.int64), pos, np.zeros(L0), qh, SCALE,
                            L0 - n_rep, protect_from, row_dtype="bf16", choose=follow)
        assert len(res["pairs"]) == n_rep
    print(f"prefill merge with exact ties: merges {list(nm)}", flush=True)

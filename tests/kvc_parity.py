"""Lockstep parity between the HIP decode step and the CPU oracle.

Each checked step copies the GPU pre-state of the sampled scopes to the host,
runs the oracle on exactly those bytes, runs the GPU step, copies the
post-state back and compares:
  * evicted sets: equal size; they may differ only in tokens whose oracle
    utility lies within 1e-6 (relative) of the cut, the largest evicted utility;
  * outputs o and lse: 2e-3 absolute for bf16 caches; 1e-5 relative (per head,
    against the head's largest |o|) for fp32 caches;
  * scores s and utilities m: 1e-5 relative + 1e-12 (all dtypes);
  * moments: n exact; S, s_k, s_v within 1e-5 of the summed magnitudes;
  * compaction: every surviving position keeps its exact row bits and vote.
The run then continues from the GPU state, so a legitimate near-tie flip does
not cascade.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc


def bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor: bf16 as uint16 bit patterns, other dtypes as they are."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32(x) -> float:
    return float(np.float32(x))


class DeviceRun:
    """A workload's cache on the GPU plus the buffers one decode step needs."""

    def __init__(self, wl: synth.Workload, capacity=None, moments=None, device="cuda", max_len=0, flags=True):
        """flags: the step reports the evicted flags (evict_out); without them a merge-mode step on
        the split path leaves the selection to the merge kernels."""
        self.wl = wl
        t = synth.cache_tensors(wl, device, capacity=capacity)
        self.scales = t["scales"]
        self.cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"], votes=t["votes"])
        self.mom = kvc.Moments.zeros(wl.n_scopes, wl.units_per_scope, wl.d, device) if (
            wl.moments if moments is None else moments) else None
        self.G = wl.G
        S, U, C = wl.n_scopes, wl.units_per_scope, self.cache.capacity
        self.out = torch.empty((S, U, wl.G, wl.d), device=device)
        self.lse = torch.empty((S, U, wl.G), device=device)
        self.s = torch.empty((S, C), device=device)
        self.evict = torch.zeros((S, C), dtype=torch.uint8, device=device) if flags else None
        self.ws = kvc.workspace(kvc.kvc_decode_workspace_size(self.cache, wl.G, max_len), device)
        self.scale = f32(1.0 / np.sqrt(wl.d))
        self.alpha = f32(wl.alpha)
        self.max_len = max_len
        self.t = wl.context   # position of the next appended token

    def inputs(self, step):
        return synth.step_inputs(self.wl, step, self.scales, self.cache.k.device)

    def step(self, step, q, kn, vn, refresh=True, merge=None, max_len=None):
        ml = self.max_len if max_len is None else max_len
        kvc.kvc_decode_step(self.cache, kn, vn, self.t, q, self.G, self.scale, self.wl.rule, self.alpha,
                            self.wl.budget, self.out, self.lse, self.s, self.mom, merge, self.evict,
                            refresh=refresh, max_len=ml, ws=self.ws)
        self.t += 1

    # ---------------------------------------------------------- host snapshots
    def snapshot(self, scopes):
        c = self.cache
        idx = torch.as_tensor(scopes, device=c.k.device, dtype=torch.long)
        lens = c.length.cpu().numpy()
        snap = {"len": lens[scopes], "k": bits(c.k[idx]), "v": bits(c.v[idx]), "pos": bits(c.pos[idx]),
                "m": bits(c.m[idx]), "votes": None if c.votes is None else bits(c.votes[idx])}
        if self.mom is not None:
            snap.update(n=bits(self.mom.n[idx]), sk=bits(self.mom.sk[idx]), sv=bits(self.mom.sv[idx]),
                        S=bits(self.mom.S[idx]))
        return snap


def oracle_state(snap, j, dtype):
    L = int(snap["len"][j])
    votes = snap["votes"][j, :L].astype(np.int64) if snap["votes"] is not None else np.ones(L, dtype=np.int64)
    return oracle.ScopeState(K=oracle.to_f64(snap["k"][j, :, :L], dtype), V=oracle.to_f64(snap["v"][j, :, :L], dtype),
                             votes=votes, pos=snap["pos"][j, :L].astype(np.int64),
                             m=snap["m"][j, :L].astype(np.float64))


def check_step(run: DeviceRun, scopes, pre, post, q, kn, vn, t, refresh=True, merge=False, report=None,
               protect_from=None):
    """Compare one GPU step on `scopes` with the oracle run on the GPU pre-state (protect_from:
    the selection's protection bound, for InertiaKV's third lazy alternative)."""
    wl = run.wl
    dtype = wl.dtype
    out = bits(run.out[torch.as_tensor(scopes, device=run.out.device)])
    lse = bits(run.lse[torch.as_tensor(scopes, device=run.out.device)])
    s_gpu = bits(run.s[torch.as_tensor(scopes, device=run.out.device)])
    ev_gpu = None if run.evict is None else bits(run.evict[torch.as_tensor(scopes, device=run.out.device)])
    qh, knh, vnh = bits(q), bits(kn), bits(vn)
    prm = oracle.StepParams(scale=run.scale, rule=wl.rule, alpha=run.alpha, budget=wl.budget,
                            score=refresh, merge=merge, row_dtype=dtype, protect_from=protect_from)
    stats = {"max_do": 0.0, "max_dlse": 0.0, "max_rel_s": 0.0, "max_rel_m": 0.0, "near_tie_flips": 0}
    for j, sc in enumerate(scopes):
        st = oracle_state(pre, j, dtype)
        L0 = st.length
        post_ref, res = oracle.decode_step(st, oracle.to_f64(knh[sc], dtype), oracle.to_f64(vnh[sc], dtype), t,
                                           oracle.to_f64(qh[sc], dtype), prm)
        L = L0 + 1
        pos_all = np.append(st.pos, t)
        # ---- outputs
        o_ref, lse_ref = res.o, res.lse
        do = np.abs(out[j].astype(np.float64) - o_ref)
        dl = np.abs(lse[j].astype(np.float64) - lse_ref)
        if dtype == "bf16":
            assert do.max() <= 2e-3, f"scope {sc}: |do| {do.max()}"
            assert dl.max() <= 2e-3, f"scope {sc}: |dlse| {dl.max()}"
        else:
            ref_inf = np.abs(o_ref).max(axis=-1, keepdims=True)
            assert np.all(do <= 1e-5 * ref_inf), f"scope {sc}: rel do {(do / ref_inf).max()}"
            assert np.all(dl <= 1e-5 * np.abs(lse_ref) + 1e-6), f"scope {sc}: dlse {dl.max()}"
        stats["max_do"] = max(stats["max_do"], float(do.max()))
        stats["max_dlse"] = max(stats["max_dlse"], float(dl.max()))
        # ---- scores
        if refresh:
            s_ref = res.s[0]
            ds = np.abs(s_gpu[j, :L].astype(np.float64) - s_ref)
            assert np.all(ds <= 1e-5 * np.abs(s_ref) + 1e-12), f"scope {sc}: rel ds {(ds / (np.abs(s_ref) + 1e-30)).max()}"
            stats["max_rel_s"] = max(stats["max_rel_s"], float((ds / (np.abs(s_ref) + 1e-30)).max()))
        # ---- evicted set
        E_ref = set(res.evicted_pos[0].tolist())
        Lp = int(post["len"][j])
        ppos = post["pos"][j, :Lp].astype(np.int64)
        E_gone = set(pos_all.tolist()) - set(ppos.tolist())      # positions the step removed
        if ev_gpu is not None:
            E_gpu = set(pos_all[ev_gpu[j, :L].astype(bool)].tolist())
            assert E_gpu == E_gone, f"scope {sc}: flagged {sorted(E_gpu)} but removed {sorted(E_gone)}"
        else:
            E_gpu = E_gone
        ev_slots = [i for i in range(L) if int(pos_all[i]) in E_gpu]
        assert len(E_gpu) == len(E_ref), f"scope {sc}: |E| {len(E_gpu)} vs {len(E_ref)}"
        m_ref = dict(zip(res.m_pos[0].tolist(), res.m_pre[0].tolist()))
        if E_ref != E_gpu:
            cut = max(m_ref[p] for p in E_ref)
            for p in E_ref ^ E_gpu:
                assert abs(m_ref[p] - cut) <= 1e-6 * abs(cut), (
                    f"scope {sc}: evict sets differ at pos {p} (m {m_ref[p]!r}, cut {cut!r})")
                stats["near_tie_flips"] += 1
        # ---- survivors: length, positions, utilities, rows, votes
        assert Lp == L - len(E_gpu), f"scope {sc}: len {Lp} vs {L - len(E_gpu)}"
        alive = sorted(set(pos_all.tolist()) - E_gpu)
        assert sorted(ppos.tolist()) == alive, f"scope {sc}: surviving positions differ"
        merged_pos = None
        if merge and res.merges[0]:
            merged_pos = _check_merge(run, sc, j, st, post_ref, res, pre, post, E_gpu, t, knh[sc], vnh[sc], stats)
        keep_m = ppos != (merged_pos if merged_pos is not None else -1)
        pm = post["m"][j, :Lp].astype(np.float64)[keep_m]
        mref = np.array([m_ref[p] for p in ppos[keep_m]])
        dm = np.abs(pm - mref)
        assert np.all(dm <= 1e-5 * np.abs(mref) + 1e-12), f"scope {sc}: rel dm {(dm / (np.abs(mref) + 1e-30)).max()}"
        stats["max_rel_m"] = max(stats["max_rel_m"], float((dm / (np.abs(mref) + 1e-30)).max()))
        slot_of = {p: i for i, p in enumerate(st.pos.tolist())}
        krows_pre = pre["k"][j]
        vrows_pre = pre["v"][j]
        for i, p in enumerate(ppos.tolist()):
            if p == merged_pos:
                continue
            if p == t:
                kr, vr = knh[sc], vnh[sc]
            else:
                kr, vr = krows_pre[:, slot_of[p]], vrows_pre[:, slot_of[p]]
            assert np.array_equal(post["k"][j][:, i], kr) and np.array_equal(post["v"][j][:, i], vr), (
                f"scope {sc}: row of pos {p} changed")
            if pre["votes"] is not None:
                exp_vote = 1 if p == t else int(pre["votes"][j, slot_of[p]])
                assert int(post["votes"][j, i]) == exp_vote
        # ---- moments: fold of the GPU's own evicted rows into the GPU pre-state
        if run.mom is not None:
            Eg = ev_slots
            Kall = np.concatenate([oracle.to_f64(pre["k"][j][:, :L0], dtype), oracle.to_f64(knh[sc], dtype)[:, None]], 1)
            Vall = np.concatenate([oracle.to_f64(pre["v"][j][:, :L0], dtype), oracle.to_f64(vnh[sc], dtype)[:, None]], 1)
            mom_pre = {"n": 0, "sk": pre["sk"][j].astype(np.float64), "sv": pre["sv"][j].astype(np.float64),
                       "S": pre["S"][j].astype(np.float64)}
            ref = oracle.fold_moments(mom_pre, Kall[:, Eg], Vall[:, Eg])
            mag_S = np.abs(pre["S"][j]).astype(np.float64) + np.einsum(
                "uea,ueb->uab", np.abs(Vall[:, Eg]), np.abs(Kall[:, Eg]))
            assert np.all(post["n"][j] == pre["n"][j] + len(Eg))
            assert np.all(np.abs(post["S"][j] - ref["S"]) <= 1e-5 * mag_S + 1e-6), f"scope {sc}: S"
            mag_k = np.abs(pre["sk"][j]) + np.abs(Kall[:, Eg]).sum(axis=1)
            mag_v = np.abs(pre["sv"][j]) + np.abs(Vall[:, Eg]).sum(axis=1)
            assert np.all(np.abs(post["sk"][j] - ref["sk"]) <= 1e-5 * mag_k + 1e-6), f"scope {sc}: sk"
            assert np.all(np.abs(post["sv"][j] - ref["sv"]) <= 1e-5 * mag_v + 1e-6), f"scope {sc}: sv"
    if report is not None:
        for key, val in stats.items():
            counts = ("near_tie_flips", "partner_tie_flips", "merged_rows_exact")
            report[key] = report.get(key, 0) + val if key in counts else max(report.get(key, 0), val)
    return stats


def _check_merge(run, sc, j, st, post_ref, res, pre, post, E_gpu, t, kn_bits, vn_bits, stats):
    """The ZIP merge of one scope (KeepKV eqs. (7), (10), (12)): the GPU's partner c is the
    oracle's unless the two cosines tie within 1e-6; merged rows agree with the oracle's
    bf16-rounded rows within one bf16 ulp, votes add exactly, utilities add. Returns the
    position whose row the merge rewrote (skipped by the row-identity check)."""
    dtype = run.wl.dtype
    pe_ref, pc_ref, _ = res.merges[0]
    Lp = int(post["len"][j])
    ppos = post["pos"][j, :Lp].astype(np.int64)
    pvotes = post["votes"][j, :Lp].astype(np.int64)
    pre_votes = np.append(pre["votes"][j, :st.length].astype(np.int64), 1)
    pos_all = np.append(st.pos, t)
    vote_of = dict(zip(pos_all.tolist(), pre_votes.tolist()))
    grown = [p for p, v in zip(ppos.tolist(), pvotes.tolist()) if v != vote_of[p]]
    assert len(grown) == 1, f"scope {sc}: {len(grown)} entries changed vote"
    pc = grown[0]
    (pe,) = tuple(E_gpu)
    assert int(pvotes[ppos.tolist().index(pc)]) == vote_of[pc] + vote_of[pe]
    if pe != pe_ref:
        stats["near_tie_flips"] += 0     # already counted by the evicted-set check
        return pc
    if pc != pc_ref:
        K = np.concatenate([oracle.to_f64(pre["k"][j][0, :st.length], dtype),
                            oracle.to_f64(kn_bits[0], dtype)[None]], 0)
        cos = K @ K[list(pos_all).index(pe)] / (np.linalg.norm(K, axis=1) + 1e-300)
        cg, cr = cos[list(pos_all).index(pc)], cos[list(pos_all).index(pc_ref)]
        assert abs(cg - cr) <= 1e-6 * abs(cr), f"scope {sc}: merge partner {pc} vs {pc_ref}"
        stats["partner_tie_flips"] = stats.get("partner_tie_flips", 0) + 1
        return pc
    i_gpu = ppos.tolist().index(pc)
    i_ref = post_ref.pos.tolist().index(pc)
    for name, ref_rows in (("k", post_ref.K), ("v", post_ref.V)):
        got = oracle.to_f64(post[name][j][:, i_gpu], dtype)
        want = ref_rows[:, i_ref]
        ulp = np.abs(want) * (2.0 ** -7 if dtype == "bf16" else 2.0 ** -23) + 1e-30
        assert np.all(np.abs(got - want) <= ulp), f"scope {sc}: merged {name} row off by >1 ulp"
        stats["merged_rows_exact"] = stats.get("merged_rows_exact", 0) + int(np.array_equal(got, want))
    m_got = float(post["m"][j, i_gpu])
    m_want = float(post_ref.m[i_ref])
    assert abs(m_got - m_want) <= 1e-5 * abs(m_want) + 1e-12, f"scope {sc}: merged utility"
    return pc


def lockstep(run: DeviceRun, steps, scopes_for_step, refresh_for_step=lambda t: True, merge=None,
             max_len_for_step=lambda t: None):
    """Run `steps` decode steps; check the ones for which scopes_for_step(step) is non-empty."""
    report = {}
    for step in range(1, steps + 1):
        q, kn, vn = run.inputs(step)
        scopes = scopes_for_step(step)
        t = run.t
        refresh = refresh_for_step(step)
        if scopes:
            pre = run.snapshot(scopes)
        mg = kvc.merge_desc(q, run.G, run.scale) if merge else None
        run.step(step, q, kn, vn, refresh=refresh, merge=mg, max_len=max_len_for_step(step))
        if scopes:
            torch.cuda.synchronize()
            post = run.snapshot(scopes)
            check_step(run, scopes, pre, post, q, kn, vn, t, refresh=refresh, merge=bool(merge), report=report)
    assert kvc.kvc_workspace_status(run.ws) == 0
    return report

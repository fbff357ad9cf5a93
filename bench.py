#!/usr/bin/env python3
"""Benchmark of the fused decode-attend-score-evict step on one MI355X.

Workload (default): one Llama-3.1-8B-shaped layer (32 query / 8 KV heads,
d = 128, bf16 cache) at 32K context compressed to a 10% budget (3276 slots
per KV head), stacked over the model's 32 layers so one launch per step
covers 256 KV heads; EMA utility (alpha 0.9) and MomentKV moments on. The
first decode step (bulk compression of 32769 -> 3276 per head) runs before
the timed region; every timed step attends over 3277 live tokens per head,
scores them, updates the utility, evicts one token per head, folds it into
the moments and compacts.

Prints one JSON line. `value` is cached tokens attended+scored+evicted per
second (live K/V rows the step processes, summed over KV heads); inputs of
every step are resident in HBM before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import synth  # noqa: E402
from compressed_decode_attention_gqa_amd import kvc  # noqa: E402
from compressed_decode_attention_gqa_amd import roofline as rf  # noqa: E402

METRIC = "cached tokens attended+scored+evicted/sec and % peak HBM GB/s at 32K ctx"
# Untimed warm-up runs the requested steps and then keeps going until this much time of
# back-to-back steps has passed: under sustained load the step time settles some 8% below
# that of the first steps (clocks ramp up over the first few hundred steps, and drop again
# after a pause), and a decode loop runs sustained.
MIN_WARMUP_S = 0.25
KERNEL_SOURCES = ["decode_unit.hip", "kvc_stream.h", "kvc_epilogue.h", "kvc_ops.h", "kvc_device.h", "kvc_decode.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_c2x32_traffic.json")


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "compressed_decode_attention_gqa_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on this workload and the current kernel source; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != kernel_source_sha() or not t.get("workload", "").startswith(workload + " "):
        return None
    return t.get("hbm_bytes_per_launch")


def host_scopes(cache, scopes, dtype, q, kn, vn):
    """Host copies of some scopes' current state and of the next step's inputs, as oracle input."""
    import oracle

    def h(x):
        x = x.detach().cpu()
        return x.view(torch.int16).numpy().view(np.uint16) if x.dtype == torch.bfloat16 else x.numpy()
    lens = cache.length.cpu().numpy()
    states = []
    for sc in scopes:
        L = int(lens[sc])
        votes = (h(cache.votes[sc, :L]).astype(np.int64) if cache.votes is not None
                 else np.ones(L, dtype=np.int64))
        states.append(oracle.ScopeState(K=oracle.to_f64(h(cache.k[sc, :, :L]), dtype),
                                        V=oracle.to_f64(h(cache.v[sc, :, :L]), dtype), votes=votes,
                                        pos=h(cache.pos[sc, :L]).astype(np.int64),
                                        m=h(cache.m[sc, :L]).astype(np.float64)))
    conv = lambda x: [oracle.to_f64(h(x[sc]), dtype) for sc in scopes]
    return states, conv(q), conv(kn), conv(vn)


def _oracle_scope_state(wl, j: int):
    """A steady-state scope of the workload built on the host (the recipe of synth: key
    scales, K/V rows, step inputs; utilities set to small positive values, moments zero) for
    timing the oracle. Returns (state, new_k, new_v, q, position) as float64 arrays."""
    import oracle
    U, d, L = wl.units_per_scope, wl.d, wl.budget
    seed = wl.seed * 1000 + j
    scales = synth.key_scales(U, d, seed, "cpu") if wl.key_scales else None
    K, V = synth.kv_rows(U, L, d, wl.dtype, seed, "cpu", scales)
    conv = lambda x: oracle.to_f64(x.view(torch.int16).numpy().view(np.uint16), "bf16") \
        if x.dtype == torch.bfloat16 else x.double().numpy()
    rng = np.random.default_rng(seed)
    votes = (1 + rng.poisson(2.0, L)).astype(np.int64) if wl.prior_votes else np.ones(L, dtype=np.int64)
    mom = {"n": 0, "sk": np.zeros((U, d)), "sv": np.zeros((U, d)), "S": np.zeros((U, d, d))} if wl.moments else None
    st = oracle.ScopeState(K=conv(K), V=conv(V), votes=votes, pos=np.arange(L, dtype=np.int64),
                           m=rng.random(L) / L, moments=mom)
    q = conv(synth.step_query(1, U, wl.G, d, wl.dtype, seed, "cpu"))
    kn, vn = synth.step_new_kv(1, U, d, wl.dtype, seed, "cpu", scales)
    return st, conv(kn), conv(vn), q, wl.context


def _oracle_worker(task):
    """One host thread (BLAS limited to one thread) running the oracle's steady decode step on
    its own scope for `seconds`; returns (steps, tokens, seconds)."""
    name, j, seconds = task
    import oracle
    from threadpoolctl import threadpool_limits
    wl = synth.WORKLOADS[name]
    st, kn, vn, q, t = _oracle_scope_state(wl, j)
    prm = oracle.StepParams(scale=float(np.float32(1 / np.sqrt(wl.d))), rule=wl.rule,
                            alpha=float(np.float32(wl.alpha)), budget=wl.budget,
                            groups=wl.n_layers if wl.scope == "model" else 1, merge=wl.merge,
                            row_dtype=wl.dtype)
    steps = tokens = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds or steps == 0:
            oracle.decode_step(st, kn, vn, t, q, prm)
            steps += 1
            tokens += scope_tokens(wl, st.length + 1)
        return steps, tokens, time.perf_counter() - t0


def cpu_baseline_pool(wl, seconds: float):
    """The float64 oracle's steady decode step on the host, run before the GPU is touched:
    one thread alone for a third of `seconds`, then one single-threaded worker process per
    core (at most 16, the host share of one GPU; 4 for the large model-scope states) for the
    rest, each on its own scope of the workload. value = tokens/s of the workers together."""
    import multiprocessing as mp
    nproc = os.cpu_count() or 1
    workers = min(nproc, 4 if wl.scope == "model" else 16)
    st1, tk1, dt1 = _oracle_worker((wl.name, 0, seconds / 3))
    with mp.get_context("spawn").Pool(workers) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_worker, [(wl.name, j, seconds * 2 / 3) for j in range(workers)])
        wall = time.perf_counter() - t0
    steps = sum(r[0] for r in res)
    tokens = sum(r[1] for r in res)
    span = max(r[2] for r in res)
    what = ("per-sequence steady steps (all layers, one slot set)" if wl.scope == "model"
            else "per-KV-head steady steps")
    return {"value": tokens / span, "unit": "tokens/s", "cores": workers, "nproc": nproc, "kind": "oracle",
            "single_thread": {"value": tk1 / dt1, "unit": "tokens/s", "cores": 1, "steps": st1},
            "sample": f"{steps} {what} of {wl.name} (L={wl.budget + 1}, G={wl.G}, k=1, "
                      f"moments {'on' if wl.moments else 'off'}{', ZIP merge' if wl.merge else ''}) in "
                      f"{span:.1f} s on {workers} worker processes with one BLAS thread each "
                      f"(pool wall {wall:.1f} s incl. start-up), numpy float64 oracle; single thread: "
                      f"{st1} steps in {dt1:.1f} s; host scopes built from the workload's recipe"}


def warm_up(call, n_min: int, min_seconds: float = MIN_WARMUP_S, chunk: int = 256) -> int:
    """Runs call(j) for j = 0, 1, ... back to back: at least n_min calls, and on until
    min_seconds have passed (the host waits for the GPU once every `chunk` calls, a gap too
    short to lower the clocks); returns the number of calls."""
    done = 0
    t0 = time.perf_counter()
    while True:
        n = min(chunk, n_min - done) if done < n_min else chunk
        for _ in range(max(1, n)):
            call(done)
            done += 1
        torch.cuda.synchronize()
        if done >= n_min and time.perf_counter() - t0 >= min_seconds:
            return done


def read_ceiling(dev, nbytes: int, reps: int = 20):
    """Streaming-read rate of the library's read probe (GB/s): the best over grid sizes of
    (a) rereading one buffer of nbytes (as the decode step rereads its cache), (b) reading
    four such buffers in turn (nothing left in the memory-side cache) and (c) one buffer read
    alternately forwards and backwards (the decode step's walk order)."""
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b in bufs:
        b.fill_(1)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for mode in ("same", "rotate", "zigzag"):
        best = 0.0
        for wg in (256, 512, 1024, 2048, 4096):
            for j in range(4):
                kvc.kvc_read_probe(bufs[0], wg, sink)
            torch.cuda.synchronize()
            e0.record()
            for j in range(reps):
                b = bufs[j % 4] if mode == "rotate" else bufs[0]
                kvc.kvc_read_probe(b, wg, sink, reverse=(mode == "zigzag" and j % 2 == 1))
            e1.record()
            torch.cuda.synchronize()
            best = max(best, nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9)
        out[mode] = best
    del bufs
    return out


def scope_tokens(wl, L: int) -> int:
    """Cached tokens one steady step of one scope attends over: every unit's live rows; with
    one slot set shared by the layers, layer 1 sees L and evicts one, the others see L - 1."""
    if wl.scope == "model":
        return wl.n_kv * (L + (wl.n_layers - 1) * (L - 1))
    return L


def step_bytes(wl, L: int) -> int:
    """Algorithmic bytes of one steady step over the whole workload (L = live tokens of a scope
    after the append). Per KV head: rf.unit_step_bytes (K/V, utility, score, q, o, append, one
    moved row, moment fold); a ZIP merge adds the cosine pass over the scope's keys and the
    merged rows; with one slot set per sequence every layer's call reads and rewrites the
    shared utility and score and only layer 1 appends and moves."""
    elem = 2 if wl.dtype == "bf16" else 4
    d, G, row = wl.d, wl.G, wl.d * (2 if wl.dtype == "bf16" else 4)
    if wl.scope == "model":
        total = 0
        for layer in range(wl.n_layers):
            Ll = L if layer == 0 else L - 1
            per_scope = (wl.n_kv * Ll * 2 * row + Ll * (12 + (4 if wl.prior_votes else 0))
                         + wl.n_kv * (G * row + G * d * 4 + G * 4))
            if layer == 0:
                U = wl.n_layers * wl.n_kv
                per_scope += U * 4 * row + 12 + U * 4 * row + 24
            total += per_scope * wl.n_scopes
        return total
    ub = rf.unit_step_bytes(L=L, k=1, G=G, d=d, elem=elem, votes=wl.prior_votes, moments=wl.moments,
                            write_score=True)
    extra = (L * row + 6 * row) if wl.merge else 0
    return (ub.total + extra) * wl.n_scopes * wl.units_per_scope


LAPROX_STAGES = ["gram", "window_pass1", "row_combine", "window_pass2", "value_norms", "product",
                 "normalise"]


def laprox_cpu_baseline(lw, inp, scale, seconds: float):
    """The fp64 oracle's per-unit LaProx work (column norms and value-output norms) timed on
    the host over as many units of the workload as fit in `seconds`."""
    import oracle
    from threadpoolctl import threadpool_info
    G = lw.H // lw.n_kv
    t0 = time.perf_counter()
    units = 0
    while time.perf_counter() - t0 < seconds and units < lw.n_layers * lw.n_kv:
        l, h = divmod(units, lw.n_kv)
        f = lambda x: x.float().cpu().numpy().astype(np.float64)
        Qw = f(inp["q_win"][l, h * G:(h + 1) * G])
        oracle.window_column_norms(Qw, f(inp["k"][l, h]), scale)
        oracle.value_output_norms(f(inp["v"][l, h]), f(inp["w_o"][l, h * G:(h + 1) * G]))
        units += 1
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": units * lw.N / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{units} KV heads of {lw.name} (N={lw.N}, G={G}, w={lw.w}, D={lw.D}): column norms "
                      f"and value-output norms in {dt:.1f} s, numpy float64 oracle (device-to-host "
                      f"copies of each head's inputs inside the timed loop)"}


def run_laprox(args):
    lw = synth.LAPROX_WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    inp = synth.laprox_inputs(lw, dev)
    units = lw.n_layers * lw.n_kv
    G = lw.H // lw.n_kv
    scale = float(np.float32(1 / np.sqrt(lw.d)))
    score = torch.empty((lw.n_layers, lw.n_kv, lw.N), dtype=torch.float32, device=dev)
    ws = kvc.workspace(kvc.kvc_laprox_workspace_size(lw.n_layers, lw.H, lw.n_kv, lw.N, lw.w, lw.d, lw.D), dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(len(LAPROX_STAGES) + 1)]
    for e in marks:
        e.record()

    def call(ev=None):
        kvc.kvc_laprox_score(inp["q_win"], inp["k"], inp["v"], inp["w_o"], lw.n_layers, lw.H, lw.n_kv, lw.N,
                             lw.w, lw.d, lw.D, scale, score, ws, events=ev)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms_per_call = start.elapsed_time(end) / args.steps
    stage_ms = np.zeros(len(LAPROX_STAGES))
    for _ in range(args.steps):
        call(marks)
        torch.cuda.synchronize()
        stage_ms += [marks[i].elapsed_time(marks[i + 1]) for i in range(len(LAPROX_STAGES))]
    stage_ms /= args.steps
    R = G * lw.w
    logit_flops = 2.0 * R * lw.N * lw.d * units                  # one window pass
    gram_flops = 2.0 * lw.d * lw.d * lw.D * units                # M = W_bar W_bar^T per unit
    r2_flops = (2.0 * lw.d * lw.d + 2.0 * lw.d) * lw.N * units   # v M v^T per token
    stages = {}
    for name, ms in zip(LAPROX_STAGES, stage_ms):
        stages[name] = {"ms": float(ms)}
    for name in ("window_pass1", "window_pass2"):
        ach = logit_flops / (stages[name]["ms"] / 1e3) / 1e12
        stages[name].update(bound="mfma", achieved=ach, peak=rf.MI355X_FP64_TFLOPS, unit="TFLOP/s",
                            frac=ach / rf.MI355X_FP64_TFLOPS, flops="2 R N d per unit, float64 MFMA")
    for name, fl, what in (("gram", gram_flops, "2 d^2 D per unit (W_bar W_bar^T), float64 MFMA"),
                           ("value_norms", r2_flops, "(2 d^2 + 2 d) N per unit (v M v^T), float64 MFMA")):
        ach = fl / (stages[name]["ms"] / 1e3) / 1e12
        stages[name].update(bound="mfma", achieved=ach, peak=rf.MI355X_FP64_TFLOPS, unit="TFLOP/s",
                            frac=ach / rf.MI355X_FP64_TFLOPS, flops=what)
    dom = max(("window_pass1", "window_pass2", "value_norms"), key=lambda n: stages[n]["ms"])
    d = stages[dom]
    result = {
        "metric": "LaProx prefill: tokens scored/sec (model-wide scores of every layer and KV head)",
        "value": units * lw.N / (ms_per_call / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_call, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 inputs; f64 MFMA logits and value norms", "data": "synthetic",
        "config": {"workload": lw.name, "layers": lw.n_layers, "q_heads": lw.H, "kv_heads": lw.n_kv,
                   "head_dim": lw.d, "hidden": lw.D, "prompt": lw.N, "window": lw.w,
                   "keep_total": lw.keep_total, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
                     "unit": d["unit"], "frac": d["frac"], "traffic": None, "launch_ms": d["ms"]},
        "stages": stages,
    }
    # the plan's measure of the value-output norms: the explicit product V W_bar (N x d times
    # d x D per unit) on bf16 MFMA; the Gram form computes the same norms with 2 d^2 per token
    vw_flops = 2.0 * lw.N * lw.d * lw.D * units
    result["value_norm_terms"] = {
        "explicit_vw_flops": vw_flops, "gram_form_flops": gram_flops + r2_flops,
        "effective_TFLOPs_value_norm_stages": vw_flops / ((stages["gram"]["ms"] + stages["value_norms"]["ms"]) / 1e3) / 1e12,
        "effective_TFLOPs_whole_call": vw_flops / (ms_per_call / 1e3) / 1e12,
        "bf16_dense_peak_TFLOPs": rf.MI355X_BF16_TFLOPS,
        "note": "explicit V W_bar flops over the measured times, against the dense bf16 peak the explicit "
                "product would run at; the Gram form reaches the same norms with about d/D of those flops, in float64"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = laprox_cpu_baseline(lw, inp, scale, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def run_moment_correct(args):
    """MomentKV corrected output over every KV head of the workload, with steady-state
    statistics (n_e = context + 1 - budget evictions folded); inputs resident in HBM."""
    import oracle
    wl = synth.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    units = wl.n_scopes * wl.units_per_scope
    G, d = wl.G, wl.d
    g = torch.Generator(device=dev).manual_seed(wl.seed)
    n_e = wl.context + 1 - wl.budget
    mom = kvc.Moments(n=torch.full((wl.n_scopes, wl.units_per_scope), n_e, dtype=torch.int32, device=dev),
                      sk=torch.randn((wl.n_scopes, wl.units_per_scope, d), generator=g, device=dev) * n_e ** 0.5,
                      sv=torch.randn((wl.n_scopes, wl.units_per_scope, d), generator=g, device=dev) * n_e ** 0.5,
                      S=torch.randn((wl.n_scopes, wl.units_per_scope, d, d), generator=g, device=dev) * n_e ** 0.5)
    q = torch.randn((units, G, d), generator=g, device=dev).to(synth.torch_dtype(wl.dtype))
    fR = torch.randn((units, G, d), generator=g, device=dev)
    lseR = torch.randn((units, G), generator=g, device=dev) + 8.0
    out = torch.empty_like(fR)
    scale = float(np.float32(1 / np.sqrt(d)))

    def call():
        kvc.kvc_moment_correct(mom, units, q, G, scale, fR, lseR, out)

    for _ in range(args.warmup):
        call()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    esz = 2 if wl.dtype == "bf16" else 4
    per_unit = d * d * 4 + 2 * d * 4 + 4 + G * d * esz + 2 * G * d * 4 + G * 4
    achieved = per_unit * units / (ms / 1e3) / 1e9
    result = {"metric": "MomentKV corrected outputs/sec (query heads corrected per second)",
              "value": units * G / (ms / 1e3), "unit": "heads/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "f64 arithmetic, fp32 statistics", "data": "synthetic",
              "config": {"workload": wl.name + " corrected output", "units": units, "G": G, "n_e": n_e},
              "roofline": {"bound": "hbm", "achieved": achieved, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                           "frac": achieved / rf.MI355X_HBM_GBPS, "traffic": None, "launch_ms": ms,
                           "bytes_per_launch": per_unit * units}}
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        done = 0
        S_h, sk_h, sv_h = mom.S.cpu().double().numpy(), mom.sk.cpu().double().numpy(), mom.sv.cpu().double().numpy()
        qh, fh, lh = q.float().cpu().double().numpy(), fR.cpu().double().numpy(), lseR.cpu().double().numpy()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            u = done % units
            sc, uu = divmod(u, wl.units_per_scope)
            oracle.corrected_output(fh[u], lh[u], qh[u], {"n": n_e, "sk": sk_h[sc, uu], "sv": sv_h[sc, uu],
                                                           "S": S_h[sc, uu]}, scale)
            done += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": done * G / dt, "unit": "heads/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{done} units of {wl.name} (G={G}) in {dt:.1f} s, numpy float64"}
    print(json.dumps(result), flush=True)


def run_moment_evict(args):
    """MomentKV moment-informed eviction at the decode steady state: every KV head holds
    budget + 1 tokens and evicts the one of lowest alpha ||r|| against the moment model, then
    folds it into its sums (kvc_moment_evict: score kernel + pick/fold kernel). Inputs resident
    in HBM; the sums keep growing by one token per repetition, which leaves the work unchanged."""
    import oracle
    from oracle.moment_evict import moment_scores
    name = args.workload if args.workload.startswith("m1_") else "m1_momentkv_llama8b_32layers_b1024"
    wl = synth.WORKLOADS[name]
    dev = "cuda"
    torch.cuda.set_device(0)
    S, d, B = wl.n_scopes, wl.d, wl.budget
    L = B + 1
    scales = synth.key_scales(S, d, wl.seed, dev) if wl.key_scales else None
    K, V = synth.kv_rows(S, L, d, wl.dtype, wl.seed, dev, scales)
    pos = torch.arange(L, dtype=torch.int32, device=dev).repeat(S, 1).contiguous()
    cache = kvc.Cache(k=K.view(S, 1, L, d).contiguous(), v=V.view(S, 1, L, d).contiguous(), pos=pos,
                      m=torch.zeros((S, L), device=dev), length=torch.full((S,), L, dtype=torch.int32, device=dev))
    n_e = wl.context - B
    ms = synth.moment_sums(S, d, n_e, wl.seed, dev)
    mom = kvc.Moments(ms["n"].view(S, 1).contiguous(), ms["sk"].view(S, 1, d).contiguous(),
                      ms["sv"].view(S, 1, d).contiguous(), ms["S"].view(S, 1, d, d).contiguous())
    alpha = synth.token_weights(S, L, wl.seed, dev)
    evict = torch.zeros((S, L), dtype=torch.uint8, device=dev)
    ws = kvc.workspace(kvc.kvc_moment_evict_workspace_size(cache), dev)
    scale = float(np.float32(1 / np.sqrt(d)))

    def call():
        kvc.kvc_moment_evict(cache, mom, alpha, scale, B, evict, max_len=L, ws=ws)

    for _ in range(args.warmup):
        call()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        call()
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / args.steps
    flops = rf.moment_evict_flops(S, L, d)
    achieved = flops / (ms_step / 1e3) / 1e12
    result = {"metric": "MomentKV moment-scored tokens/sec (live tokens scored, one eviction per head)",
              "value": S * L / (ms_step / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "f64", "data": "synthetic",
              "config": {"workload": wl.name + " steady eviction", "heads": S, "live_tokens_per_head": L,
                         "budget": B, "n_e": n_e, "cache": wl.dtype},
              "roofline": {"bound": "mfma", "achieved": achieved, "peak": rf.MI355X_FP64_TFLOPS, "unit": "TFLOP/s",
                           "frac": achieved / rf.MI355X_FP64_TFLOPS, "traffic": None, "launch_ms": ms_step,
                           "flops_per_launch": flops}}
    if not args.no_cpu_baseline:
        Kh = oracle.to_f64(K.view(torch.int16).cpu().numpy().view(np.uint16), wl.dtype) if wl.dtype == "bf16" \
            else K.cpu().double().numpy()
        Vh = oracle.to_f64(V.view(torch.int16).cpu().numpy().view(np.uint16), wl.dtype) if wl.dtype == "bf16" \
            else V.cpu().double().numpy()
        ah = alpha.cpu().double().numpy()
        mh = {k: v.cpu().double().numpy() for k, v in ms.items()}
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            sc = done % S
            moment_scores(Kh[sc], Vh[sc], ah[sc], {"n": n_e, "sk": mh["sk"][sc], "sv": mh["sv"][sc],
                                                   "S": mh["S"][sc]}, scale)
            done += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": done * L / dt, "unit": "tokens/s", "cores": torch.get_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"{done} heads of {wl.name} (L={L}) scored in {dt:.1f} s, numpy float64"}
    print(json.dumps(result), flush=True)


def run_ema_init(args):
    """KeepKV's window initialisation of the EMA utility at the end of a 4k prompt for every KV
    head (kvc_keepkv_ema_init): 32 window queries (the page's w = 31) per KV head, G = 4 query
    heads, alpha 0.9. Events are recorded between the four kernels of each call."""
    from oracle.keepkv_ema_init import ema_window_init
    import oracle
    wl = synth.WORKLOADS["k1_keepkv_prefill_llama8b_4k"]
    dev = "cuda"
    torch.cuda.set_device(0)
    S, d, G, N, n_win, alpha = wl.n_scopes, wl.d, wl.G, wl.context, 32, 0.9
    t = synth.cache_tensors(wl, dev)
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"])
    q = synth.window_queries(S, G, n_win, d, wl.seed, dev).contiguous()
    scale = float(np.float32(1 / np.sqrt(d)))
    ws = kvc.workspace(kvc.kvc_keepkv_ema_init_workspace_size(cache, G, n_win, N), dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in marks:
        e.record()   # torch creates the event at its first record
    for _ in range(args.warmup):
        kvc.kvc_keepkv_ema_init(cache, q, G, n_win, N, scale, alpha, ws)
    torch.cuda.synchronize()
    stages = []
    for _ in range(args.steps):
        kvc.kvc_keepkv_ema_init(cache, q, G, n_win, N, scale, alpha, ws, events=marks)
        torch.cuda.synchronize()
        stages.append([marks[i].elapsed_time(marks[i + 1]) for i in range(4)])
    st = np.median(np.array(stages), axis=0)
    ms = float(st.sum())
    # each window pass: 2 G n_win N d flops per head on the fp64 MFMA
    pass_flops = S * 2.0 * G * n_win * N * d
    ach = pass_flops / (st[2] / 1e3) / 1e12
    result = {"metric": "KeepKV EMA window initialisation: prompt tokens scored/sec",
              "value": S * N / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16 cache; f64 logits and softmax statistics", "data": "synthetic",
              "config": {"workload": wl.name, "heads": S, "prompt": N, "window": n_win, "G": G, "alpha": alpha},
              "roofline": {"bound": "mfma", "achieved": ach, "peak": rf.MI355X_FP64_TFLOPS, "unit": "TFLOP/s",
                           "frac": ach / rf.MI355X_FP64_TFLOPS, "traffic": None, "kernel": "k_lap_window<4, 2>",
                           "launch_ms": float(st[2]), "flops_per_launch": pass_flops},
              "stages_ms": {"window_pass1": float(st[0]), "row_combine": float(st[1]),
                            "window_pass2": float(st[2]), "block_sum": float(st[3])}}
    if not args.no_cpu_baseline:
        Kh = oracle.to_f64(t["k"][0, 0, :N].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        qh = oracle.to_f64(q[0].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < min(args.cpu_seconds, 10.0):
            ema_window_init(qh, Kh, scale, alpha)
            reps += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": reps * N / dt, "unit": "tokens/s", "cores": torch.get_num_threads(),
                                  "kind": "oracle",
                                  "sample": f"{reps} window initialisations of one KV head ({N} tokens, {n_win} "
                                            f"window queries) in {dt:.1f} s, numpy float64 oracle"}
    print(json.dumps(result), flush=True)


def run_prefill_merge(args):
    """KeepKV prefill compression of every KV head: greedy all-pairs ZIP merging from the prompt
    length down to the budget, the last 32 positions protected (kvc_keepkv_prefill_merge). The
    cache is restored from an HBM copy before each repetition; events bracket the call alone."""
    from oracle.keepkv_prefill import prefill_merge
    import oracle
    wl = synth.WORKLOADS["k1_keepkv_prefill_llama8b_4k"]
    dev = "cuda"
    torch.cuda.set_device(0)
    S, d, B, L0 = wl.n_scopes, wl.d, wl.budget, wl.context
    protect_from = L0 - 32
    t = synth.cache_tensors(wl, dev)
    votes = torch.ones((S, L0 + 1), dtype=torch.int32, device=dev)
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"], votes=votes)
    q = synth.step_query(0, S, wl.G, d, wl.dtype, wl.seed, dev).contiguous()
    merge = kvc.merge_desc(q, wl.G, float(np.float32(1 / np.sqrt(d))))
    saved = [x.clone() for x in (cache.k, cache.v, cache.votes, cache.pos, cache.m, cache.length)]
    fields = (cache.k, cache.v, cache.votes, cache.pos, cache.m, cache.length)
    evict = torch.zeros((S, cache.capacity), dtype=torch.uint8, device=dev)
    n_merged = torch.zeros((S,), dtype=torch.int32, device=dev)
    ws = kvc.workspace(kvc.kvc_keepkv_prefill_workspace_size(cache), dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for e in marks:
        e.record()   # torch creates the event at its first record
    stages = []   # per repetition: key norms and flags, initial lists, merge loop (ms)
    for rep in range(args.warmup + args.steps):
        for x, y in zip(fields, saved):
            x.copy_(y)
        torch.cuda.synchronize()
        kvc.kvc_keepkv_prefill_merge(cache, merge, B, protect_from, evict, None, n_merged, ws=ws, events=marks)
        torch.cuda.synchronize()
        if rep >= args.warmup:
            stages.append([marks[i].elapsed_time(marks[i + 1]) for i in range(3)])
    if kvc.kvc_workspace_status(ws) != 0 or int(n_merged.min()) != L0 - B:
        raise SystemExit("prefill merge did not reach the budget")
    st = np.median(np.array(stages), axis=0)
    ms = float(st.sum())
    # algorithmic bytes of the merge loop (the dominant kernel): each merge reads the keys of the
    # candidates other than the merged pair once, to get their cosines with the merged key
    cand0, es = protect_from, 2 if wl.dtype == "bf16" else 4
    loop_bytes = S * sum((cand0 - t - 2) * d * es for t in range(L0 - B))
    ach = loop_bytes / (st[2] / 1e3) / 1e9
    rows_flops = S * 2.0 * cand0 * cand0 * d
    result = {"metric": "KeepKV prefill compression: prompt tokens compressed/sec (greedy all-pairs ZIP merging)",
              "value": S * L0 / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16 cache; f64 cosines and merge weights", "data": "synthetic",
              "config": {"workload": wl.name, "heads": S, "prompt": L0, "budget": B, "protected": L0 - protect_from,
                         "merges_per_head": L0 - B, "G": wl.G},
              "roofline": {"bound": "hbm", "achieved": ach, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                           "frac": ach / rf.MI355X_HBM_GBPS, "traffic": None, "kernel": "k_pm_loop",
                           "launch_ms": float(st[2]), "bytes_per_launch": loop_bytes},
              "stages_ms": {"prep": float(st[0]), "initial_lists": float(st[1]), "merge_loop": float(st[2])},
              "initial_lists_fp64_tflops": rows_flops / (st[1] / 1e3) / 1e12}
    if not args.no_cpu_baseline:
        # the oracle on one head, for a bounded number of merges
        sc = 0
        Kh = oracle.to_f64(saved[0][sc, 0, :L0].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        Vh = oracle.to_f64(saved[1][sc, 0, :L0].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        qh = oracle.to_f64(q[sc].view(torch.int16).cpu().numpy().view(np.uint16), "bf16")
        n_steps = 12
        t0 = time.perf_counter()
        prefill_merge(Kh, Vh, np.ones(L0, dtype=np.int64), np.arange(L0), np.zeros(L0), qh,
                      float(np.float32(1 / np.sqrt(d))), L0 - n_steps, protect_from, row_dtype="bf16")
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n_steps / dt * L0 / (L0 - B), "unit": "tokens/s",
                                  "cores": torch.get_num_threads(), "kind": "oracle",
                                  "sample": f"the first {n_steps} merges of one head (L0={L0}) in {dt:.1f} s, "
                                            "numpy float64 oracle, scaled to whole prompts per second"}
    print(json.dumps(result), flush=True)


def run_refresh(args):
    """KeepKV's periodic refresh at k1's shape after T = 64 decode steps (kvc_keepkv_refresh_marked):
    the full KV of 256 heads x 4160 tokens reloaded from pinned host memory, the EMA state restarted
    over the last 32 steps' queries, greedy ZIP merging back to the budget (the last 32 positions
    protected), compaction. Events between the four stages; the cache holds an unrelated state
    before each repetition (the refresh overwrites it). Repetitions: at most one warm-up and five
    timed (a call takes about a third of a second)."""
    import oracle
    wl = synth.WORKLOADS["k1_keepkv_prefill_llama8b_4k"]
    dev = "cuda"
    torch.cuda.set_device(0)
    S, d, G, B, L0 = wl.n_scopes, wl.d, wl.G, wl.budget, wl.context
    T, n_win = 64, 32
    n = L0 + T
    protect_from = n - 32
    scale, alpha = float(np.float32(1 / np.sqrt(d))), float(np.float32(0.9))
    # the full KV in pinned host memory
    Kf, Vf = synth.kv_rows(S, n, d, "bf16", wl.seed, "cpu", synth.key_scales(S, d, wl.seed, "cpu"))
    hk = torch.empty((S, n, d), dtype=torch.bfloat16, pin_memory=True)
    hv = torch.empty((S, n, d), dtype=torch.bfloat16, pin_memory=True)
    hp = torch.empty((S, n), dtype=torch.int32, pin_memory=True)
    hk.copy_(Kf)
    hv.copy_(Vf)
    hp.copy_(torch.arange(n, dtype=torch.int32).repeat(S, 1))
    del Kf, Vf
    # the cache: capacity n, holding an unrelated compressed state
    cache = kvc.Cache(k=torch.zeros((S, 1, n, d), dtype=torch.bfloat16, device=dev),
                      v=torch.zeros((S, 1, n, d), dtype=torch.bfloat16, device=dev),
                      pos=torch.zeros((S, n), dtype=torch.int32, device=dev),
                      m=torch.zeros((S, n), device=dev), length=torch.full((S,), B, dtype=torch.int32, device=dev),
                      votes=torch.ones((S, n), dtype=torch.int32, device=dev))
    q_win = torch.stack([synth.step_query(L0 + T - n_win + 1 + j, S, G, d, "bf16", wl.seed, dev)
                         for j in range(n_win)], dim=2).contiguous()
    q_ref = q_win[:, :, -1, :].contiguous()
    merge = kvc.merge_desc(q_ref, G, scale)
    n_merged = torch.zeros((S,), dtype=torch.int32, device=dev)
    ws = kvc.workspace(kvc.kvc_keepkv_refresh_workspace_size(cache, G, n_win, n), dev)
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
    for e in marks:
        e.record()
    stages = []   # reload, EMA restart, merging, compaction (ms)
    warm, reps = min(args.warmup, 1), max(1, min(args.steps, 5))
    for rep in range(warm + reps):
        cache.length.fill_(B)
        torch.cuda.synchronize()
        kvc.kvc_keepkv_refresh(cache, hk, hv, hp, n, q_win, n_win, merge, alpha, B, protect_from, None, n_merged,
                               ws=ws, events=marks)
        torch.cuda.synchronize()
        if rep >= warm:
            stages.append([marks[i].elapsed_time(marks[i + 1]) for i in range(4)])
    if kvc.kvc_workspace_status(ws) != 0 or int(n_merged.min()) != n - B or int(cache.length.max()) != B:
        raise SystemExit("refresh did not reach the budget")
    st = np.median(np.array(stages), axis=0)
    ms = float(st.sum())
    reload_bytes = 2 * S * n * d * 2 + S * n * 4
    loop_bytes = S * sum((protect_from - t - 2) * d * 2 for t in range(n - B))
    ach = loop_bytes / (st[2] / 1e3) / 1e9
    result = {"metric": "KeepKV periodic refresh: tokens reloaded and recompressed/sec",
              "value": S * n / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": reps, "warmup": warm,
              "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16 cache; f64 logits, cosines and merge weights", "data": "synthetic",
              "config": {"workload": wl.name, "heads": S, "refresh_period": T, "tokens": n, "window": n_win,
                         "budget": B, "protected": n - protect_from, "G": G},
              "roofline": {"bound": "hbm", "achieved": ach, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                           "frac": ach / rf.MI355X_HBM_GBPS, "traffic": None, "kernel": "k_pm_loop",
                           "launch_ms": float(st[2]), "bytes_per_launch": loop_bytes},
              "stages_ms": {"reload_h2d": float(st[0]), "ema_restart": float(st[1]), "merging": float(st[2]),
                            "compaction": float(st[3])},
              "reload": {"bytes": reload_bytes, "GBps": reload_bytes / (st[0] / 1e3) / 1e9,
                         "share_of_refresh": float(st[0] / ms)}}
    if not args.no_cpu_baseline:
        # the oracle's refresh of one head, bounded to its first 12 merges (the window restart in full)
        h = lambda x: x.view(torch.int16).numpy().view(np.uint16)
        Kh = oracle.to_f64(h(hk[0]), "bf16")
        Vh = oracle.to_f64(h(hv[0]), "bf16")
        qw = oracle.to_f64(h(q_win[0].cpu()), "bf16")
        qr = oracle.to_f64(h(q_ref[0].cpu()), "bf16")
        n_steps = 12
        t0 = time.perf_counter()
        oracle.refresh(Kh, Vh, np.arange(n), qw, qr, scale, alpha, n - n_steps, protect_from, row_dtype="bf16")
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": n_steps / dt * n / (n - B), "unit": "tokens/s",
                                  "cores": torch.get_num_threads(), "kind": "oracle",
                                  "sample": f"the window restart and the first {n_steps} merges of one head "
                                            f"(n={n}) in {dt:.1f} s, numpy float64 oracle, scaled to whole "
                                            "refreshes per second"}
    print(json.dumps(result), flush=True)


def run_first_step(args):
    """The first decode step after prefill: attend and score over the whole context, then
    compress every KV head to its budget (k = context + 1 - budget evictions per head: select,
    moment fold, compaction). The cache is restored from an HBM copy before each repetition;
    only the step call itself is inside the events."""
    wl = synth.WORKLOADS[args.workload]
    dev = "cuda"
    torch.cuda.set_device(0)
    S, U, G, d, B = wl.n_scopes, wl.units_per_scope, wl.G, wl.d, wl.budget
    t = synth.cache_tensors(wl, dev)
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"], votes=t["votes"])
    mom = kvc.Moments.zeros(S, U, d, dev) if wl.moments else None
    out = torch.empty((S, U, G, d), device=dev)
    lse = torch.empty((S, U, G), device=dev)
    s = torch.empty((S, cache.capacity), device=dev)
    evict = torch.zeros((S, cache.capacity), dtype=torch.uint8, device=dev)
    ws = kvc.workspace(kvc.kvc_decode_workspace_size(cache, G, 0), dev)
    scale = float(np.float32(1 / np.sqrt(d)))
    alpha = float(np.float32(wl.alpha))
    fields = [cache.k, cache.v, cache.pos, cache.m, cache.length] + ([cache.votes] if cache.votes is not None else [])
    saved = [x.clone() for x in fields]
    q, kn, vn = synth.step_inputs(wl, 1, t["scales"], dev)
    L0 = wl.initial_len + 1
    times = []
    for rep in range(args.warmup + args.steps):
        for x, y in zip(fields, saved):
            x.copy_(y)
        if mom is not None:
            for x in (mom.n, mom.sk, mom.sv, mom.S):
                x.zero_()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        kvc.kvc_decode_step(cache, kn, vn, wl.context, q, G, scale, wl.rule, alpha, B, out, lse, s, mom, None,
                            evict, max_len=L0, ws=ws)
        end.record()
        torch.cuda.synchronize()
        if rep >= args.warmup:
            times.append(start.elapsed_time(end))
    assert int(cache.length.min()) == B and int(cache.length.max()) == B
    status = kvc.kvc_workspace_status(ws)
    if status != 0:
        raise SystemExit(f"device status {status} after the first step")
    ms = float(np.median(times))
    k = L0 - B
    esz = 2 if wl.dtype == "bf16" else 4
    row = 2 * d * esz
    ev = evict[:, :L0].bool()
    moved = int((~ev[:, B:]).sum())                       # survivors above the budget fill the holes
    per_token = row + 12 + 8 + (4 if wl.prior_votes else 0)   # K/V, m r/w + s, select keys, votes
    bytes_step = (S * U * L0 * row + S * L0 * (per_token - row)
                  + S * U * k * row                       # evicted rows re-read by the fold
                  + moved * (2 * U * row + 24)            # moved rows and slot arrays (read + write)
                  + (S * U * (2 * d * d * 4 + 4 * d * 4) if wl.moments else 0))
    achieved = bytes_step / (ms / 1e3) / 1e9
    result = {"metric": "first decode step: cached tokens attended+scored, compressed to the budget, per sec",
              "value": S * U * L0 / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
              "config": {"workload": wl.name + " first step", "kv_heads": S * U, "live_tokens_per_head": L0,
                         "budget": B, "evicted_per_head": k, "moved_rows": moved, "moments": wl.moments},
              "roofline": {"bound": "hbm", "achieved": achieved, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                           "frac": achieved / rf.MI355X_HBM_GBPS, "traffic": None, "bytes_per_step": bytes_step,
                           "ms_all": times}}
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        for x, y in zip(fields, saved):
            x.copy_(y)
        prm = oracle.StepParams(scale=scale, rule=wl.rule, alpha=alpha, budget=B)
        states, qh, knh, vnh = host_scopes(cache, [0], wl.dtype, q, kn, vn)
        t0 = time.perf_counter()
        done = 0
        while time.perf_counter() - t0 < min(args.cpu_seconds, 20.0) or done == 0:
            oracle.decode_step(states[0], knh[0], vnh[0], wl.context, qh[0], prm)
            done += 1
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        result["cpu_baseline"] = {"value": done * U * L0 / dt, "unit": "tokens/s", "cores": int(threads),
                                  "kind": "oracle",
                                  "sample": f"{done} first steps of KV head 0 of {wl.name} (L={L0}, k={k}) "
                                            f"in {dt:.1f} s, numpy float64 oracle"}
    print(json.dumps(result), flush=True)


def run_stream_ceiling(args):
    """The streaming-read ceiling alone: the library's read probe over one decode step's
    algorithmic bytes of the headline workload (and over 1 GiB), every grid size and order."""
    wl = synth.WORKLOADS["c2x32_llama8b_32layers_32k"]
    torch.cuda.set_device(0)
    nbytes = step_bytes(wl, wl.budget + 1)
    res = {"step_bytes": read_ceiling("cuda", nbytes, reps=50), "1GiB": read_ceiling("cuda", 1 << 30, reps=20)}
    best = max(max(v.values()) for v in res.values())
    print(json.dumps({"metric": "streaming-read ceiling (read probe)", "value": best, "unit": "GB/s",
                      "n_gpus": 1, "higher_is_better": True, "detail": res,
                      "peak": rf.MI355X_HBM_GBPS, "frac_of_peak": best / rf.MI355X_HBM_GBPS}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2x32_llama8b_32layers_32k")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--op", default="step", choices=["step", "first_step", "moment_correct", "moment_evict", "prefill_merge", "refresh",
                                                     "ema_init", "stream_ceiling"],
                    help="step: the fused decode step (default); first_step: the bulk compression step "
                         "after prefill; moment_correct: MomentKV's corrected output")
    ap.add_argument("--model-path", default="groups", choices=["groups", "per_layer"],
                    help="model-scope workloads: the layers after the first in one kvc_decode_groups call, "
                         "or one call per layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-read probe after the timed steps")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the graph-replayed timing of per-head workloads after the timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference kernel for counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs the decode step on a single "
              "MI355X; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.op == "stream_ceiling":
        return run_stream_ceiling(args)
    if args.op == "moment_evict":
        return run_moment_evict(args)
    if args.op == "ema_init":
        return run_ema_init(args)
    if args.op == "prefill_merge":
        return run_prefill_merge(args)
    if args.op == "refresh":
        return run_refresh(args)
    if args.op == "moment_correct":
        run_moment_correct(args)
        return
    if args.op == "first_step":
        if args.steps == 200 and args.warmup == 20:
            args.steps, args.warmup = 5, 1
        run_first_step(args)
        return
    if args.workload in synth.LAPROX_WORKLOADS:
        if args.steps == 200 and args.warmup == 20:
            args.steps, args.warmup = 5, 1
        run_laprox(args)
        return
    wl = synth.WORKLOADS[args.workload]
    # the oracle's rate on the host cores, measured before the GPU is touched
    cpu_base = None if args.no_cpu_baseline else cpu_baseline_pool(wl, args.cpu_seconds)
    dev = "cuda"
    torch.cuda.set_device(0)
    S, U, G, d, B = wl.n_scopes, wl.units_per_scope, wl.G, wl.d, wl.budget
    t = synth.cache_tensors(wl, dev)
    cache = kvc.Cache(k=t["k"], v=t["v"], pos=t["pos"], m=t["m"], length=t["length"], votes=t["votes"])
    mom = kvc.Moments.zeros(S, U, d, dev) if wl.moments else None
    out = torch.empty((S, U, G, d), device=dev)
    lse = torch.empty((S, U, G), device=dev)
    s = torch.empty((S, cache.capacity), device=dev)
    ws = kvc.workspace(kvc.kvc_decode_workspace_size(cache, G, 0), dev)
    scale = float(np.float32(1 / np.sqrt(d)))
    alpha = float(np.float32(wl.alpha))
    n_steps = 1 + args.warmup + args.steps
    q_all, kn_all, vn_all = [], [], []
    for step in range(1, n_steps + 1):
        q, kn, vn = synth.step_inputs(wl, step, t["scales"], dev)
        q_all.append(q)
        kn_all.append(kn)
        vn_all.append(vn)
    pos_next = [wl.context]                     # the next token's position (prior entries lie below it)
    n_calls = [0]

    def next_pos():
        t = pos_next[0]
        pos_next[0] += 1
        n_calls[0] += 1
        return t

    if wl.scope == "model":
        # the first layer's call appends every layer's rows, attends, scores, updates the
        # shared utility and evicts to the budget; the later layers cannot evict: one
        # kvc_decode_groups call for all of them (utility chain in closed form), or with
        # --model-path per_layer one kvc_decode_step per layer with budget = capacity
        nkv = wl.n_kv
        cap = cache.capacity
        nl = wl.n_layers
        q_first = [q[:, :nkv].contiguous() for q in q_all]
        q_rest = [q[:, nkv:].contiguous() for q in q_all]
        q_layers = [[q[:, l * nkv:(l + 1) * nkv].contiguous() for l in range(1, nl)] for q in q_all] \
            if args.model_path == "per_layer" else None
        out_first = torch.empty((S, nkv, G, d), device=dev)
        lse_first = torch.empty((S, nkv, G), device=dev)
        out_rest = torch.empty((S, (nl - 1) * nkv, G, d), device=dev)
        lse_rest = torch.empty((S, (nl - 1) * nkv, G), device=dev)
        # per-layer calls write [S][nkv][G][d] contiguously: one buffer per layer
        out_layers = [torch.empty((S, nkv, G, d), device=dev) for _ in range(1, nl)] if q_layers else None
        lse_layers = [torch.empty((S, nkv, G), device=dev) for _ in range(1, nl)] if q_layers else None

        def step_call(i, max_len):
            refresh = wl.lazy_refresh == 0 or n_calls[0] % wl.lazy_refresh == 0
            t = next_pos()
            kvc.kvc_decode_step(cache, kn_all[i], vn_all[i], t, q_first[i], G, scale, wl.rule, alpha, B,
                                out_first, lse_first, s, mom, None, None, refresh=refresh, attn_unit0=0,
                                attn_units=nkv, max_len=max_len, ws=ws)
            if nl == 1:
                return
            if q_layers is None:
                kvc.kvc_decode_groups(cache, q_rest[i], G, scale, wl.rule, alpha, nkv, nl - 1, nkv, out_rest,
                                      lse_rest, s, refresh=refresh, max_len=max_len, ws=ws)
                return
            for l in range(1, nl):
                kvc.kvc_decode_step(cache, None, None, t, q_layers[i][l - 1], G, scale, wl.rule, alpha, cap,
                                    out_layers[l - 1], lse_layers[l - 1], s,
                                    mom, None, None, refresh=refresh, attn_unit0=l * nkv, attn_units=nkv,
                                    max_len=max_len, ws=ws)
    else:
        merges = [kvc.merge_desc(q, G, scale) for q in q_all] if wl.merge else None

        def step_call(i, max_len):
            kvc.kvc_decode_step(cache, kn_all[i], vn_all[i], next_pos(), q_all[i], G, scale, wl.rule, alpha, B,
                                out, lse, s, mom, merges[i] if merges else None, None, max_len=max_len, ws=ws)

    step_call(0, wl.initial_len + 1)            # first step: bulk compression to the budget
    # the requested warm-up steps, then on (cycling through their inputs) until the GPU has run
    # MIN_WARMUP_S of back-to-back steps
    warm = lambda j: step_call(1 + j % max(1, args.warmup), B + 1)
    warm_steps = warm_up(warm, args.warmup, chunk=256 if wl.scope != "model" else 16)

    # The timed region is K back-to-back steps on the launch stream (torch's current
    # stream), bracketed by two HIP events: for the per-head workloads a step is one
    # kernel launch, so the region's length over K is that kernel's average duration
    # (events between launches would add their own cost to every step); a model-scope
    # step is one call per layer. A last run of warm-up steps is queued right before the
    # start event, so the GPU does not idle (and drop its clocks) between warm-up and timing.
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for j in range(256 if wl.scope != "model" else 16):
        warm(j)
        warm_steps += 1
    start.record()
    for j in range(args.steps):
        step_call(1 + args.warmup + j, B + 1)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    launch_ms = total_ms / args.steps
    assert int(cache.length.min()) == B and int(cache.length.max()) == B
    status = kvc.kvc_workspace_status(ws)
    if status != 0:
        raise SystemExit(f"device status {status} after the timed steps")

    L = B + 1
    tokens_per_step = S * scope_tokens(wl, L) if wl.scope == "model" else S * U * L
    ms_per_step = total_ms / args.steps
    value = tokens_per_step / (ms_per_step / 1e3)
    bytes_per_launch = step_bytes(wl, L)
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    traffic = measured_traffic(wl.name)
    result = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "warmup_steps_run": warm_steps, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "layers": wl.n_layers, "batch": wl.batch, "kv_heads": wl.n_kv,
                   "q_heads": wl.n_kv * G, "head_dim": d, "context": wl.context, "budget": B,
                   "live_tokens_per_head": L, "rule": wl.rule, "alpha": wl.alpha, "moments": wl.moments,
                   "logits": "f64 accumulate", "values": "f32 accumulate", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": rf.MI355X_HBM_GBPS, "unit": "GB/s",
                     "frac": achieved / rf.MI355X_HBM_GBPS, "traffic": traffic,
                     "bytes_per_launch": bytes_per_launch, "launch_ms": launch_ms,
                     "wall_GBps": bytes_per_launch / (ms_per_step / 1e3) / 1e9},
    }
    # The same steps replayed from a captured HIP graph (64 steps with their own inputs and
    # positions; replays repeat them): the step's GPU time without per-call host submission,
    # which bounds the eager rate of the latency-bound shapes. Reported beside the eager value.
    if wl.scope != "model" and not args.no_graph:
        gsteps = 64
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for j in range(gsteps):
                step_call(1 + args.warmup + j % max(1, args.steps), B + 1)
        for _ in range(3):
            graph.replay()
        replays = max(3, args.steps // gsteps)
        start.record()
        for _ in range(replays):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        g_ms = start.elapsed_time(end) / (replays * gsteps)
        assert int(cache.length.min()) == B and int(cache.length.max()) == B
        if kvc.kvc_workspace_status(ws) != 0:
            raise SystemExit("device status after the graph replays")
        result["graph"] = {"ms_per_step": g_ms, "value": tokens_per_step / (g_ms / 1e3), "steps_per_graph": gsteps,
                           "replays": replays}
    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        y.copy_(x)
        torch.cuda.synchronize()
    if not args.no_ceiling:
        ceil = read_ceiling(dev, bytes_per_launch)
        result["roofline"]["measured_ceiling_GBps"] = max(ceil.values())
        result["roofline"]["measured_ceiling"] = {k: round(v, 1) for k, v in ceil.items()}
        result["roofline"]["frac_of_measured_ceiling"] = achieved / max(ceil.values())
    if cpu_base is not None:
        result["cpu_baseline"] = cpu_base
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()

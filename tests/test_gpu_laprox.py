"""GPU parity of kvc_laprox_score and the model-wide Top-K (MI355X).

Scores are compared with the fp64 oracle on the same bf16 bytes: relative
1e-5 (+1e-12); keep sets may differ only in tokens whose oracle score lies
within 1e-6 (relative) of the cut. The full-size prefill (36 layers x 8 KV
heads, 65536 tokens, w = 32, D = 4096) is checked on every property that
holds at any size and, for one whole layer, against the oracle token by token.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from synth.workloads import LaproxWorkload

pytestmark = pytest.mark.gpu

C5 = synth.LAPROX_WORKLOADS["c5_laprox_qwen3_8b_64k"]


def _say(*a):
    print(*a, flush=True)


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _run(lw, inp, scale):
    score = torch.empty((lw.n_layers, lw.n_kv, lw.N), dtype=torch.float32, device="cuda")
    ws = kvc.workspace(kvc.kvc_laprox_workspace_size(lw.n_layers, lw.H, lw.n_kv, lw.N, lw.w, lw.d, lw.D))
    kvc.kvc_laprox_score(inp["q_win"], inp["k"], inp["v"], inp["w_o"], lw.n_layers, lw.H, lw.n_kv, lw.N,
                         lw.w, lw.d, lw.D, scale, score, ws)
    return score


def _gpu_keep(score, K):
    """Model-wide Top-K on the device: evict the bottom n - K by (score, flat index)."""
    flat = score.reshape(1, -1).contiguous()
    n = flat.shape[1]
    evict = torch.zeros((1, n), dtype=torch.uint8, device="cuda")
    ws = kvc.workspace(kvc.kvc_select_workspace_size(1, n))
    kvc.kvc_select_evict(flat, None, None, 1, n, K, evict, None, ws)
    return evict.cpu().numpy()[0] == 0


def _check_keep(keep_gpu, s_ref, K):
    keep_ref = oracle.laprox_keep(s_ref, K).reshape(-1)
    assert keep_gpu.sum() == K
    diff = np.flatnonzero(keep_gpu != keep_ref)
    if diff.size:
        cut = np.sort(s_ref.reshape(-1))[-K]
        assert np.all(np.abs(s_ref.reshape(-1)[diff] - cut) <= 1e-6 * cut), (diff[:8], cut)
    return diff.size


@pytest.mark.parametrize("n_layers,H,n_kv,N,w,D", [
    (2, 8, 2, 700, 8, 256),       # G = 4, one ragged tile
    (1, 16, 2, 2500, 16, 128),    # G = 8: 128 window rows (two workgroup halves), three tiles
    (2, 4, 2, 333, 4, 64),        # G = 2
    (1, 2, 2, 1100, 8, 192),      # G = 1, one token past a tile
    (1, 32, 8, 1500, 32, 512),    # the full-size group shape: G = 4, w = 32
])
def test_laprox_matches_oracle(n_layers, H, n_kv, N, w, D):
    _say("laprox", n_layers, H, n_kv, N, w, D)
    lw = LaproxWorkload(name="t", seed=11 + N, n_layers=n_layers, H=H, n_kv=n_kv, d=128, D=D, N=N, w=w,
                        keep_per_head=max(1, N // 20))
    inp = synth.laprox_inputs(lw, "cuda")
    scale = float(np.float32(1.0 / np.sqrt(128)))
    s = _run(lw, inp, scale).cpu().numpy().astype(np.float64)
    s_ref = oracle.laprox_scores(_f64(inp["q_win"]), _f64(inp["k"]), _f64(inp["v"]), _f64(inp["w_o"]), scale)
    err = np.abs(s - s_ref) / (s_ref + 1e-300)
    assert np.all(np.abs(s - s_ref) <= 1e-5 * s_ref + 1e-12), err.max()
    np.testing.assert_allclose(s.reshape(n_layers, -1).sum(1), 1.0, rtol=1e-5)
    K = lw.keep_total
    flips = _check_keep(_gpu_keep(torch.from_numpy(s.astype(np.float32)).cuda(), K), s_ref, K)
    _say("  max rel err %.2e, keep-set flips within the tie band: %d" % (err.max(), flips))


def test_laprox_full_size_sampled():
    """36 x 8 units of 65536 tokens in one call; one layer checked against the oracle token by token."""
    lw = C5
    inp = synth.laprox_inputs(lw, "cuda")
    scale = float(np.float32(1.0 / np.sqrt(lw.d)))
    score = _run(lw, inp, scale)
    torch.cuda.synchronize()
    s = score.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(s)) and np.all(s >= 0)
    np.testing.assert_allclose(s.reshape(lw.n_layers, -1).sum(1), 1.0, rtol=1e-5)
    K = lw.keep_total
    keep = _gpu_keep(score, K)
    assert keep.sum() == K
    flat = s.reshape(-1)
    cut = flat[keep].min()
    assert flat[~keep].max() <= cut
    # one whole layer against the oracle
    l = 17
    Qw = _f64(inp["q_win"][l:l + 1])
    Kl, Vl, Wl = _f64(inp["k"][l:l + 1]), _f64(inp["v"][l:l + 1]), _f64(inp["w_o"][l:l + 1])
    s_ref = oracle.laprox_scores(Qw, Kl, Vl, Wl, scale)[0]
    got = s[l]
    assert np.all(np.abs(got - s_ref) <= 1e-5 * s_ref + 1e-12), np.max(np.abs(got - s_ref) / s_ref)
    # keep decisions of that layer under the device cut
    keep_l = keep.reshape(lw.n_layers, lw.n_kv, lw.N)[l]
    sure_keep = s_ref > cut * (1 + 1e-6)
    sure_evict = s_ref < cut * (1 - 1e-6)
    assert np.all(keep_l[sure_keep]) and not np.any(keep_l[sure_evict])
    _say("c5 layer %d: max rel err %.2e, kept in layer %d" % (l, np.max(np.abs(got - s_ref) / s_ref),
                                                               int(keep_l.sum())))

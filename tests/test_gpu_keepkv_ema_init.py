"""GPU parity of KeepKV's EMA window initialisation (kvc_keepkv_ema_init).

m[s][i] of every prompt token within 1e-5 relative (+1e-12 absolute) of the float64 oracle
(ema_window_init: the causal group-mean softmax of each window query, weighted by
(1 - alpha) alpha^(n_win - 1 - j)); slots past the prompt untouched; per-scope sums
1 - alpha^n_win. Shapes: G = 1, 2, 4, 8; window rows in one, two and four 128-row operator
blocks; prompt lengths off the 2048-token tile; capacity above the prompt; and the 4k-prompt
Llama shape in full (256 KV heads, 33 window queries), oracle on sampled heads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import bits
from oracle.keepkv_ema_init import ema_window_init

pytestmark = pytest.mark.gpu

D = 128
SCALE = float(np.float32(1.0 / np.sqrt(D)))


def _say(*a):
    print(*a, flush=True)


def _case(S, N, cap, n_win, G, alpha, seed, heads=None):
    _say("ema init", S, N, cap, n_win, G, alpha)
    scales = synth.key_scales(S, D, seed, "cuda")
    K, V = synth.kv_rows(S, cap, D, "bf16", seed, "cuda", scales)
    cache = kvc.Cache(k=K.view(S, 1, cap, D).contiguous(), v=V.view(S, 1, cap, D).contiguous(),
                      pos=torch.arange(cap, dtype=torch.int32, device="cuda").repeat(S, 1).contiguous(),
                      m=torch.full((S, cap), 7.0, dtype=torch.float32, device="cuda"),
                      length=torch.full((S,), N, dtype=torch.int32, device="cuda"))
    q = synth.window_queries(S, G, n_win, D, seed, "cuda").contiguous()   # [S][G][n_win][D]
    ws = kvc.workspace(kvc.kvc_keepkv_ema_init_workspace_size(cache, G, n_win, N))
    kvc.kvc_keepkv_ema_init(cache, q, G, n_win, N, SCALE, alpha, ws)
    torch.cuda.synchronize()
    got = cache.m.cpu().numpy().astype(np.float64)
    assert np.all(got[:, N:] == 7.0)
    np.testing.assert_allclose(got[:, :N].sum(axis=1), 1 - alpha ** n_win, rtol=1e-5)
    Kh = oracle.to_f64(bits(cache.k[:, 0]), "bf16")
    qh = oracle.to_f64(bits(q), "bf16")
    worst = 0.0
    for s in (range(S) if heads is None else heads):
        ref = ema_window_init(qh[s], Kh[s, :N], SCALE, alpha)
        err = np.abs(got[s, :N] - ref)
        assert np.all(err <= 1e-5 * ref + 1e-12), (s, float((err / np.maximum(ref, 1e-300)).max()))
        worst = max(worst, float((err / np.maximum(ref, 1e-300)).max()))
    _say("  max rel err %.2e" % worst)


@pytest.mark.parametrize("S,N,cap,n_win,G,alpha", [
    (3, 700, 720, 33, 4, 0.9),     # 132 window-head rows: two operator blocks
    (2, 2049, 2049, 5, 1, 0.8),    # one token past a tile
    (2, 300, 512, 64, 8, 0.95),    # 16 window rows per block: four blocks
    (4, 1000, 1000, 1, 2, 0.5),    # a single window query
])
def test_ema_init_matches_oracle(S, N, cap, n_win, G, alpha):
    _case(S, N, cap, n_win, G, alpha, seed=100 + N + n_win)


def test_ema_init_full_size_sampled():
    wl = synth.WORKLOADS["k1_keepkv_prefill_llama8b_4k"]
    _case(wl.n_scopes, wl.context, wl.context + 1, 33, wl.G, 0.9, seed=wl.seed, heads=[0, 1, 77, 128, 255])


def test_ema_predict_matches_oracle():
    """KeepKV eq. (14): kvc_ema_predict = m / (1 - alpha^t) on slots [0, len) of every scope
    (oracle.predicted_scores on the same m), other slots untouched; in place; and after t EMA
    updates from zero with a constant score, the prediction is that score."""
    _say("ema predict")
    rng = np.random.default_rng(17)
    S, cap = 5, 1000
    lens = torch.tensor([1000, 0, 517, 1, 999], dtype=torch.int32, device="cuda")
    m = torch.from_numpy(rng.random((S, cap)).astype(np.float32) * 1e-3).cuda()
    for alpha, t in ((0.9, 1), (0.9, 37), (0.8, 2000), (0.5, 3)):
        out = torch.full((S, cap), -5.0, device="cuda")
        kvc.kvc_ema_predict(m, lens, S, cap, alpha, t, out)
        torch.cuda.synchronize()
        got, mh = out.cpu().numpy().astype(np.float64), m.cpu().numpy()
        a32 = float(np.float32(alpha))
        for s, L in enumerate(lens.tolist()):
            ref = oracle.predicted_scores(mh[s, :L].astype(np.float64), a32, t)
            assert np.all(np.abs(got[s, :L] - ref) <= 1e-6 * ref + 1e-30), (alpha, t, s)
            assert np.all(got[s, L:] == -5.0)
    m2 = m.clone()
    kvc.kvc_ema_predict(m2, None, S, cap, 0.9, 5, m2)
    ref = oracle.predicted_scores(m.cpu().numpy().astype(np.float64), float(np.float32(0.9)), 5)
    assert np.all(np.abs(m2.cpu().numpy() - ref) <= 1e-6 * ref)
    # a constant score s: t EMA updates from zero give (1 - alpha^t) s; the prediction is s
    s_const = torch.from_numpy(rng.random((S, cap)).astype(np.float32)).cuda()
    full = torch.full((S,), cap, dtype=torch.int32, device="cuda")
    state = torch.zeros((S, cap), device="cuda")
    for t in range(1, 13):
        kvc.kvc_ema_update(state, s_const, full, S, cap, "ema", 0.9)
        pred = torch.empty_like(state)
        kvc.kvc_ema_predict(state, full, S, cap, 0.9, t, pred)
        torch.cuda.synchronize()
        assert torch.allclose(pred, s_const, rtol=2e-6, atol=0), t

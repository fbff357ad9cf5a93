"""GPU parity of kvc_moment_correct, MomentKV's normalisation-corrected output (MI355X).

Inputs are seeded synthetic rows: the evicted rows' running sums are formed
on the host in fp32, the retained output and log-partition come from the
oracle's attention; the kernel's output is compared with the oracle's
corrected output on the same fp32 values (1e-5 of the largest |output|).
A second test runs real decode steps with moments and corrects the output
of the compressed cache, against the oracle on the same state.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from compressed_decode_attention_gqa_amd import kvc
from kvc_parity import DeviceRun, bits

pytestmark = pytest.mark.gpu

C2 = synth.WORKLOADS["c2_llama8b_layer_32k"]


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype,G,U,nE", [("bf16", 4, 37, 23), ("f32", 1, 8, 5), ("bf16", 8, 5, 300),
                                          ("bf16", 2, 6, 1)])
def test_moment_correct_matches_oracle(dtype, G, U, nE):
    g = torch.Generator().manual_seed(1000 + U)
    d = 128
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn((U, G, d), generator=g).to(dt)
    KR = torch.randn((U, 50, d), generator=g).to(dt)
    VR = torch.randn((U, 50, d), generator=g).to(dt)
    KE = (torch.randn((U, nE, d), generator=g) * 0.5 + torch.randn((U, 1, d), generator=g)).to(dt)
    VE = torch.randn((U, nE, d), generator=g).to(dt)
    n = torch.full((U,), nE, dtype=torch.int32)
    n[0] = 0                                    # a unit with nothing evicted yet
    f64 = lambda t: t.double()
    sk = f64(KE).sum(1).float()
    sv = f64(VE).sum(1).float()
    S = torch.einsum("ued,uef->udf", f64(VE), f64(KE)).float()
    sk[0], sv[0], S[0] = 0, 0, 0
    scale = float(np.float32(1 / np.sqrt(d)))
    fR = np.zeros((U, G, d))
    lseR = np.zeros((U, G))
    for u in range(U):
        _, _, fR[u], lseR[u] = oracle.attend_unit(q[u].double().numpy(), KR[u].double().numpy(),
                                                  VR[u].double().numpy(), None, scale)
    lseR[1] = -np.inf                           # empty retained set: the estimate alone
    fR[1] = 0
    fR32, lse32 = torch.from_numpy(fR).float(), torch.from_numpy(lseR).float()
    mom = kvc.Moments(n=n.cuda(), sk=sk.cuda(), sv=sv.cuda(), S=S.cuda())
    out = torch.empty((U, G, d), device="cuda")
    kvc.kvc_moment_correct(mom, U, q.cuda(), G, scale, fR32.cuda(), lse32.cuda(), out)
    inplace = fR32.cuda()
    kvc.kvc_moment_correct(mom, U, q.cuda(), G, scale, inplace, lse32.cuda(), inplace)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.array_equal(got, inplace.cpu().numpy())
    for u in range(U):
        mu = {"n": int(n[u]), "sk": sk[u].double().numpy(), "sv": sv[u].double().numpy(), "S": S[u].double().numpy()}
        ref = oracle.corrected_output(fR32[u].double().numpy(), lse32[u].double().numpy(), q[u].double().numpy(),
                                      mu, scale)
        tol = 1e-5 * np.abs(ref).max() + 1e-7
        assert np.abs(got[u] - ref).max() <= tol, (u, np.abs(got[u] - ref).max())
    assert np.array_equal(got[0], fR32[0].numpy())


def test_moment_correct_after_decode_steps():
    """Decode steps with moments fold real evictions; the compressed cache's output is then
    corrected and compared with the oracle on the same state."""
    wl = C2.scaled(context=1500, budget=150, steps=4, n_kv=6, moments=True)
    run = DeviceRun(wl)
    for step in range(1, wl.steps + 1):
        run.step(step, *run.inputs(step))
    q, _, _ = run.inputs(wl.steps + 1)
    S_, U = wl.n_scopes, wl.units_per_scope
    fR = torch.empty((S_, U, wl.G, wl.d), device="cuda")
    lseR = torch.empty((S_, U, wl.G), device="cuda")
    kvc.kvc_decode_attn_score(run.cache, None, None, run.t, q, wl.G, run.scale, fR, lseR, None, 0, run.ws)
    out = torch.empty_like(fR)
    kvc.kvc_moment_correct(run.mom, S_ * U, q, wl.G, run.scale, fR, lseR, out)
    torch.cuda.synchronize()
    snap = run.snapshot(list(range(S_)))
    got = out.cpu().numpy()
    qh = bits(q)
    worst = 0.0
    for sc in range(S_):
        L = int(snap["len"][sc])
        K = oracle.to_f64(snap["k"][sc][0, :L], "bf16")
        V = oracle.to_f64(snap["v"][sc][0, :L], "bf16")
        qq = oracle.to_f64(qh[sc, 0], "bf16")
        _, _, f_R, lse_R = oracle.attend_unit(qq, K, V, None, run.scale)
        mu = {"n": int(snap["n"][sc][0]), "sk": snap["sk"][sc][0].astype(np.float64),
              "sv": snap["sv"][sc][0].astype(np.float64), "S": snap["S"][sc][0].astype(np.float64)}
        assert mu["n"] == wl.context + wl.steps - wl.budget
        ref = oracle.corrected_output(f_R, lse_R, qq, mu, run.scale)
        err = np.abs(got[sc, 0] - ref).max()
        worst = max(worst, err)
        assert err <= 2e-3, (sc, err)
    _say("moment correct after steps: max |d out| %.2e" % worst)

"""GPU parity of the decision rule at the threshold: a token is stored only when its
score exceeds tau ("Hybrid Associative Memories", App. A.1 "Forward Pass"), so a
score equal to tau stays out, and a NaN score never routes.

Two sources of exact ties are used, both independent of rounding:
- the fit-error score of the first token of a sequence that starts from a zero
  state is exactly 1 (the prediction is the zero vector, cos := 0), so tau = 1.0
  keeps it out and the float just below 1.0 lets it in, on every RNN path;
- learned-router scores (HAM_EXTERNAL_SCORES) set equal to tau, to NaN, or to the
  float just above tau, in ham_forward and in ham_decode_step.
Routing and the cache are compared with the oracle exactly; outputs at the dtype
tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs
from parity import check_forward, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
BELOW_ONE = np.nextafter(np.float32(1.0), np.float32(0.0))


@pytest.mark.parametrize("dtype,T,d,force", [(torch.bfloat16, 200, 128, False),   # chunked RNN
                                             (torch.bfloat16, 200, 64, True),     # token-serial
                                             (torch.float32, 70, 64, False)])
def test_fit_error_tie_at_the_first_token(dtype, T, d, force):
    B, H = 2, 3
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=300 + T + d)
    t = to_dev(inp, dtype, DEV)
    for tau_val, want in ((np.float32(1.0), 0), (BELOW_ONE, 1)):
        tau = np.full(H, tau_val, np.float32)
        print(f"fit-error tie: dtype={dtype} T={T} d={d} force_recurrent={force} tau={tau_val!r}", flush=True)
        out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                              scale=d ** -0.5, force_recurrent=force, want_o_rnn=True, want_o_kv=True)
        torch.cuda.synchronize()
        e = out["e"].cpu().numpy()
        r = out["routed"].cpu().numpy()
        assert np.all(e[:, 0, :] == 1.0)
        assert np.all(r[:, 0, :] == want), r[:, 0, :]
        check_forward(out, inp, tau, dtype, scale=d ** -0.5)


def _scores_with_ties(B, T, H, tau, seed):
    rng = np.random.default_rng(seed)
    rs = rng.random((B, T, H), dtype=np.float32)
    rs[:, 0::6, :] = tau                                       # exact ties: never routed
    rs[:, 1::6, :] = np.nan                                    # NaN: never routed
    rs[:, 2::6, :] = np.nextafter(tau, np.float32(np.inf))     # just above: routed
    return rs


@pytest.mark.parametrize("dtype,T,d", [(torch.bfloat16, 200, 128), (torch.float32, 130, 64)])
def test_router_ties_and_nan_forward(dtype, T, d):
    B, H = 2, 3
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=320 + T)
    tau = np.array([0.3, 0.5, 0.7], np.float32)
    rs = _scores_with_ties(B, T, H, tau, 321)
    t = to_dev(inp, dtype, DEV)
    print(f"router ties forward: dtype={dtype} T={T} d={d}", flush=True)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=d ** -0.5, router_scores=torch.from_numpy(rs).to(DEV),
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    r = out["routed"].cpu().numpy().astype(bool)
    with np.errstate(invalid="ignore"):
        want = rs > tau[None, None, :]
    assert np.array_equal(r, want)
    assert not r[:, 0::6, :].any() and not r[:, 1::6, :].any() and r[:, 2::6, :].all()
    # check_forward compares routing (exactly for router scores), the cache, the state
    # and the outputs with the oracle fed the same scores
    check_forward(out, inp, tau, dtype, scale=d ** -0.5, router_score=rs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_ties_and_nan_decode(dtype):
    B, H, d = 2, 3, 64
    T0, steps = 66, 20
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=340)
    tau = np.array([0.3, 0.5, 0.7], np.float32)
    rs = _scores_with_ties(B, T, H, tau, 341)
    scale = d ** -0.5
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, router_score=rs)
    t = to_dev(inp, dtype, DEV)
    rsd = torch.from_numpy(rs).to(DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    print(f"router ties decode: dtype={dtype} prefix={T0} steps={steps}", flush=True)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    o1 = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d, scale=scale, cap=T,
                         router_scores=rsd[:, :T0].contiguous())
    S = o1["S"]
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale)
    outs, rts = [], []
    for s in range(steps):
        tt = T0 + s
        x = {n: t[n][:, tt].contiguous() for n in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, cache["Kc"], cache["Vc"], cache["pos"],
             cache["count"], torch.full((B,), tt, dtype=torch.int32, device=DEV),
             router_scores=rsd[:, tt].contiguous())
        outs.append(np_of(plan.o)); rts.append(plan.routed.cpu().numpy())
    torch.cuda.synchronize()
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rts, 1)], 1).astype(bool)
    assert np.array_equal(r_all, ref["routed"].astype(bool))
    assert not r_all[:, 0::6, :].any() and not r_all[:, 1::6, :].any() and r_all[:, 2::6, :].all()
    cnt = cache["count"].cpu().numpy()
    assert np.array_equal(cnt, ref["count"])
    pos = cache["pos"].cpu().numpy()
    for b in range(B):
        for h in range(H):
            assert np.array_equal(pos[b, h, :cnt[b, h]], ref["pos"][b, h, :cnt[b, h]])
    assert rel_err_slices(np.stack(outs, 1), ref["o"][:, T0:], 2) < TOL[dtype]
    assert rel_err_slices(np_of(S), ref["S"], 1) < 1e-4

"""GPU: cache rows at or past a head's routed count are never read.

The forward writes rows 0 .. count-1 of each head's cache and the decode step appends
behind them; the rest of the capacity keeps whatever the caller's buffer holds.  Here
those rows hold NaN before the calls, so any read of them (a key tile row past the
last visible key that the load does not zero-fill, a decode read past the count) would
make the outputs NaN.  Sizes put the counts at ragged places inside 64-key tiles and
leave spare capacity behind the sequence.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, tau_for_rho
from parity import TOL, check_forward, check_routing, np_of, rel_err_slices, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _tau(inp, rho, scale):
    e = oracle.forward(**inp, tau=np.full(inp["q"].shape[2], np.inf, np.float32), scale=scale)["e"]
    return tau_for_rho(e, rho)


@pytest.mark.parametrize("B,T,H,dk,dv,cap,seed", [
    (1, 200, 2, 64, 64, 200, 41), (2, 129, 1, 128, 128, 320, 42), (1, 333, 1, 128, 128, 400, 43)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_forward_reads_no_row_past_the_count(B, T, H, dk, dv, cap, seed, dtype):
    inp = make_inputs(B, T, H, dk, dv, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    scale = dk ** -0.5
    tau = _tau(inp, 0.5, scale)
    t = to_dev(inp, dtype, DEV)
    plan = ham.ForwardPlan(B, T, H, dk, dv, dtype, DEV, cap=cap, scale=scale, want_o_rnn=True,
                           want_o_kv=True)
    plan.Kc.fill_(float("nan"))
    plan.Vc.fill_(float("nan"))
    plan(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV))
    torch.cuda.synchronize()
    out = plan.result()
    for name in ("o", "o_rnn", "o_kv"):
        assert torch.isfinite(out[name]).all(), name
    check_forward(out, inp, tau, dtype, scale=scale, cap=cap)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_reads_no_row_past_the_count(dtype):
    B, H, d = 2, 2, 128
    T0, steps, cap = 75, 12, 160
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=44)
    scale = d ** -0.5
    tau = _tau(inp, 0.5, scale)
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=cap)
    t = to_dev(inp, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    fplan = ham.ForwardPlan(B, T0, H, d, d, dtype, DEV, cap=cap, scale=scale)
    fplan.Kc.fill_(float("nan"))
    fplan.Vc.fill_(float("nan"))
    fplan(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d)
    o1 = fplan.result()
    S = o1["S"]
    dplan = ham.DecodePlan(B, H, d, d, cap, dtype, DEV, scale=scale)
    es, rs, os_ = [], [], []
    for s in range(steps):
        tt = T0 + s
        x = {n: t[n][:, tt].contiguous() for n in t}
        t_abs = torch.full((B,), tt, dtype=torch.int32, device=DEV)
        dplan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, o1["Kc"], o1["Vc"], o1["pos"],
              o1["count"], t_abs)
        es.append(dplan.e.cpu().numpy())
        rs.append(dplan.routed.cpu().numpy())
        os_.append(np_of(dplan.o))
    torch.cuda.synchronize()
    assert int(dplan.status.item()) == 0
    o_dec = np.stack(os_, 1)
    assert np.isfinite(o_dec).all()
    e_all = np.concatenate([o1["e"].cpu().numpy(), np.stack(es, 1)], 1)
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rs, 1)], 1)
    if check_routing(e_all, r_all, ref, tau):
        ref = oracle.forward(**inp, tau=tau, scale=scale, cap=cap, mask_override=r_all)
    assert rel_err_slices(o_dec, ref["o"][:, T0:], 2) < TOL[dtype]
    assert np.array_equal(o1["count"].cpu().numpy(), ref["count"])

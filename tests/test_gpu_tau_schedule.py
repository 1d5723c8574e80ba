"""GPU parity of per-token routing thresholds (a schedule along the sequence).

"Hybrid Associative Memories" §6: the growth of the KV cache can follow a target
schedule along the sequence, set at test time.  With HAM_TAU_PER_TOKEN the
threshold is one value per token and head ([B,T,H]; decode: [B,H] per step).
Compared with the oracle through the C ABI under the usual protocol (routing exact
outside the near-threshold band, outputs within the dtype tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, tau_for_rho
from parity import check_forward, check_routing, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _dt(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def _schedule(inp, scale, seed):
    """Thresholds that keep about 80% of the early tokens and 20% of the late ones: per
    head the quantile of the token's own position band, plus a little noise."""
    e = oracle.forward(**inp, tau=np.full(inp["q"].shape[2], INF, np.float32), scale=scale)["e"]
    B, T, H = e.shape
    rng = np.random.default_rng(seed)
    lo, hi = tau_for_rho(e, 0.8), tau_for_rho(e, 0.2)
    ramp = np.linspace(0.0, 1.0, T, dtype=np.float64)[None, :, None]
    sched = lo[None, None, :] * (1 - ramp) + hi[None, None, :] * ramp
    sched = sched + 1e-3 * rng.standard_normal((B, T, H))
    return np.ascontiguousarray(np.broadcast_to(sched, (B, T, H)).astype(np.float32))


@pytest.mark.parametrize("B,T,H,d,rec", [(2, 200, 3, 128, False), (1, 97, 2, 64, False),
                                         (2, 130, 2, 128, True)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_schedule_forward(B, T, H, d, rec, dtype):
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=150 + T)
    scale = d ** -0.5
    sched = _schedule(inp, scale, 150 + T)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(sched).to(DEV),
                          scale=scale, force_recurrent=rec, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    res = check_forward(out, inp, sched, dtype, scale=scale)
    r = out["routed"].cpu().numpy().astype(bool)
    half = T // 2
    assert r[:, :half].mean() > r[:, half:].mean()       # the schedule thins the cache out


def test_schedule_route_stats():
    B, T, H, d = 2, 300, 4, 64
    inp = make_inputs(B, T, H, d, seed=151)
    sched = _schedule(inp, 1.0, 151)
    t = to_dev(inp, torch.float32, DEV)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(sched).to(DEV),
                             near_band=1e-3)
    ref = oracle.forward(**inp, tau=sched, scale=1.0)
    check_routing(st["e"].cpu().numpy(), st["routed"].cpu().numpy(), ref, sched)
    want = oracle.route_stats(dict(ref, e=st["e"].cpu().numpy().astype(np.float64)), sched, near_band=1e-3)
    assert np.array_equal(st["n_near"].cpu().numpy(), want["n_near"])
    assert np.array_equal(st["count"].cpu().numpy(), st["routed"].cpu().numpy().sum(axis=1))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_schedule_decode_steps_equal_forward(dtype):
    B, H, d = 3, 2, 128
    T0, steps = 70, 20
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=152)
    scale = d ** -0.5
    sched = _schedule(inp, scale, 152)
    ref = oracle.forward(**inp, tau=sched, scale=scale, cap=T)
    t = to_dev(inp, dtype, DEV)
    sd = torch.from_numpy(sched).to(DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    o1 = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], sd[:, :T0].contiguous(),
                         scale=scale, cap=T)
    S = o1["S"]
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale)
    es, rs, os_ = [], [], []
    for s in range(steps):
        tt = T0 + s
        x = {n: t[n][:, tt].contiguous() for n in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], sd[:, tt].contiguous(), S, cache["Kc"],
             cache["Vc"], cache["pos"], cache["count"], torch.full((B,), tt, dtype=torch.int32, device=DEV))
        es.append(plan.e.cpu().numpy()); rs.append(plan.routed.cpu().numpy()); os_.append(np_of(plan.o))
    torch.cuda.synchronize()
    e_all = np.concatenate([o1["e"].cpu().numpy(), np.stack(es, 1)], 1)
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rs, 1)], 1)
    if check_routing(e_all, r_all, ref, sched):
        ref = oracle.forward(**inp, tau=sched, scale=scale, cap=T, mask_override=r_all)
    assert rel_err_slices(np.stack(os_, 1), ref["o"][:, T0:], 2) < TOL[dtype]
    assert np.array_equal(cache["count"].cpu().numpy(), ref["count"])

"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Sizes stay small enough for the oracle to finish in seconds while spanning several
64-token chunks, 64-query blocks and key tiles, with ragged tails.  Full-size
workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import SMALL, make_inputs, make_gates, make_workload, tau_for_rho
from parity import check_forward, check_routing, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _tau(inp, rho, scale=0.125):
    e = oracle.forward(**inp, tau=np.full(inp["q"].shape[2], INF, np.float32), scale=scale)["e"]
    return tau_for_rho(e, rho)


def _run(inp, tau, dtype, **kw):
    t = to_dev(inp, dtype, DEV)
    extra = {}
    for n in ("q_attn", "k_attn", "v_attn", "gate_rnn", "gate_kv", "S0"):
        if n in kw and kw[n] is not None:
            x = torch.from_numpy(np.ascontiguousarray(kw.pop(n)))
            extra[n] = (x.to(dtype) if n.endswith("attn") else x.float()).to(DEV)
        else:
            kw.pop(n, None)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          want_o_rnn=True, want_o_kv=True, **extra, **kw)
    torch.cuda.synchronize()
    return out


def test_small_fp32_workload():
    w = SMALL
    inp = make_workload(w)
    tau = _tau(inp, w.rho, w.attn_scale)
    out = _run(inp, tau, torch.float32, scale=w.attn_scale)
    res = check_forward(out, inp, tau, torch.float32, scale=w.attn_scale)
    rho = float(out["count"].sum()) / (w.B * w.T * w.H)
    assert abs(rho - 0.5) <= res["nflip"] / (w.B * w.T * w.H) + 1e-12
    print("small fp32 errors", res["errs"], "near flips", res["nflip"])


@pytest.mark.parametrize("B,T,H,dk,dv,seed", [
    (1, 1, 1, 64, 64, 1), (1, 37, 2, 64, 128, 2), (2, 64, 1, 128, 64, 3),
    (1, 65, 3, 128, 128, 4), (2, 200, 2, 64, 64, 5), (1, 333, 1, 128, 128, 6)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_shapes_ragged(B, T, H, dk, dv, seed, dtype):
    inp = make_inputs(B, T, H, dk, dv, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    scale = dk ** -0.5
    tau = _tau(inp, 0.5, scale)
    gr, gk = make_gates(B, T, H, seed)
    out = _run(inp, tau, dtype, scale=scale, gate_rnn=gr, gate_kv=gk)
    check_forward(out, inp, tau, dtype, scale=scale, gates=(gr, gk))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_tau_limits(dtype):
    B, T, H, d = 2, 150, 2, 128
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=21)
    scale = d ** -0.5
    out = _run(inp, np.full(H, INF, np.float32), dtype, scale=scale)
    assert int(out["count"].sum()) == 0 and int(out["routed"].sum()) == 0
    assert float(out["o_kv"].abs().max()) == 0.0
    check_forward(out, inp, np.full(H, INF, np.float32), dtype, scale=scale)
    out = _run(inp, np.full(H, -INF, np.float32), dtype, scale=scale)
    assert out["count"].cpu().tolist() == [[T] * H] * B
    check_forward(out, inp, np.full(H, -INF, np.float32), dtype, scale=scale)


def test_literal_unit_scale_and_separate_attention_inputs():
    B, T, H, d = 1, 130, 2, 64
    inp = make_inputs(B, T, H, d, seed=22)
    att = make_inputs(B, T, H, d, seed=23)
    tau = _tau(inp, 0.4, 1.0)
    out = _run(inp, tau, torch.float32, scale=1.0, q_attn=att["q"], k_attn=att["k"], v_attn=att["v"])
    check_forward(out, inp, tau, torch.float32, scale=1.0, attn=att)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_continuation_equals_one_call(dtype):
    B, T, H, d = 2, 190, 2, 64
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=24)
    scale = 0.125
    tau = _tau(inp, 0.5, scale)
    T1 = 77
    first = {n: a[:, :T1] for n, a in inp.items()}
    second = {n: a[:, T1:] for n, a in inp.items()}
    t1 = to_dev(first, dtype, DEV)
    t2 = to_dev(second, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    o1 = ham.ham_forward(t1["q"], t1["k"], t1["v"], t1["beta"], t1["g"], tau_d, scale=scale, cap=T)
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    o2 = ham.ham_forward(t2["q"], t2["k"], t2["v"], t2["beta"], t2["g"], tau_d, scale=scale,
                         S0=o1["S"].clone(), cache=cache, t0=T1, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    ref1 = oracle.forward(**first, tau=tau, scale=scale, cap=T)
    ref_cache = {n: ref1[n] for n in ("Kc", "Vc", "pos", "count")}
    check_routing(o1["e"].cpu().numpy(), o1["routed"].cpu().numpy(), ref1, tau)
    check_forward(o2, second, tau, dtype, scale=scale, S0=ref1["S"], cache=ref_cache, t0=T1)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_steps_equal_forward(dtype):
    B, H, d = 3, 2, 128
    T0, steps = 70, 24
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=25)
    scale = d ** -0.5
    tau = _tau(inp, 0.5, scale)
    gr, gk = make_gates(B, T, H, 25)
    ref = oracle.forward(**inp, tau=tau, scale=scale, gate_rnn=gr, gate_kv=gk, cap=T)
    t = to_dev(inp, dtype, DEV)
    grd, gkd = torch.from_numpy(gr).to(DEV), torch.from_numpy(gk).to(DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    o1 = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d, scale=scale,
                         cap=T, gate_rnn=grd[:, :T0].contiguous(), gate_kv=gkd[:, :T0].contiguous())
    S = o1["S"]
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale, want_o_rnn=True, want_o_kv=True)
    es, rs, os_ = [], [], []
    for s in range(steps):
        tt = T0 + s
        x = {n: t[n][:, tt].contiguous() for n in t}
        t_abs = torch.full((B,), tt, dtype=torch.int32, device=DEV)
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, cache["Kc"], cache["Vc"],
             cache["pos"], cache["count"], t_abs, gate_rnn=grd[:, tt].contiguous(),
             gate_kv=gkd[:, tt].contiguous())
        es.append(plan.e.cpu().numpy()); rs.append(plan.routed.cpu().numpy())
        os_.append(np_of(plan.o))
    torch.cuda.synchronize()
    assert int(plan.status.item()) == 0
    e_all = np.concatenate([o1["e"].cpu().numpy(), np.stack(es, 1)], 1)
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rs, 1)], 1)
    nflip = check_routing(e_all, r_all, ref, tau)
    if nflip:
        ref = oracle.forward(**inp, tau=tau, scale=scale, gate_rnn=gr, gate_kv=gk, cap=T,
                             mask_override=r_all)
    o_dec = np.stack(os_, 1)
    err = rel_err_slices(o_dec, ref["o"][:, T0:], 2)
    assert err < TOL[dtype], err
    assert np.array_equal(cache["count"].cpu().numpy(), ref["count"])
    assert rel_err_slices(np_of(S), ref["S"], 1) < 1e-4


def test_decode_capacity_flag():
    B, H, d, cap = 1, 1, 64, 4
    inp = make_inputs(B, 8, H, d, seed=26)
    t = to_dev(inp, torch.float32, DEV)
    tau_d = torch.full((H,), -float("inf"), device=DEV)
    S = torch.zeros((B, H, d, d), device=DEV)
    cache = dict(Kc=torch.zeros((B, H, cap, d), device=DEV), Vc=torch.zeros((B, H, cap, d), device=DEV),
                 pos=torch.full((B, H, cap), -1, dtype=torch.int32, device=DEV),
                 count=torch.zeros((B, H), dtype=torch.int32, device=DEV))
    plan = ham.DecodePlan(B, H, d, d, cap, torch.float32, DEV, scale=0.125)
    for s in range(6):
        x = {n: t[n][:, s].contiguous() for n in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, cache["Kc"], cache["Vc"],
             cache["pos"], cache["count"], torch.full((B,), s, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        assert int(cache["count"].item()) == min(s + 1, cap)
        assert int(plan.status.item()) == (1 if s + 1 > cap else 0)
    assert cache["pos"].cpu().tolist() == [[[0, 1, 2, 3]]]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_route_stats(dtype):
    B, T, H, d = 2, 260, 3, 128
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=27)
    tau = _tau(inp, 0.25, d ** -0.5)
    ref = oracle.forward(**inp, tau=tau, scale=d ** -0.5)
    st_ref = oracle.route_stats(ref, tau, near_band=1e-3)
    t = to_dev(inp, dtype, DEV)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                             near_band=1e-3)
    nflip = check_routing(st["e"].cpu().numpy(), st["routed"].cpu().numpy(), ref, tau)
    cnt = st["count"].cpu().numpy()
    assert np.abs(cnt - st_ref["count"]).sum() <= nflip
    assert abs(st["rho"] - st_ref["rho"]) <= nflip / (B * T * H) + 1e-12
    nn = st["n_near"].cpu().numpy()
    assert np.abs(nn - st_ref["n_near"]).sum() <= 2   # band edges may differ by rounding
    assert abs(st["rho"] - 0.25) < 0.01


def test_deterministic_bitwise():
    B, T, H, d = 2, 300, 2, 128
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=28)
    tau = _tau(inp, 0.5, d ** -0.5)
    a = _run(inp, tau, torch.bfloat16, scale=d ** -0.5)
    b = _run(inp, tau, torch.bfloat16, scale=d ** -0.5)
    for n in ("o", "o_rnn", "o_kv", "e", "routed", "S", "Kc", "Vc", "pos", "count"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunked_equals_recurrent(dtype):
    B, T, H, d = 2, 400, 2, 128
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=29)
    scale = d ** -0.5
    tau = _tau(inp, 0.5, scale)
    a = _run(inp, tau, dtype, scale=scale)
    b = _run(inp, tau, dtype, scale=scale, force_recurrent=True)
    assert float((a["e"] - b["e"]).abs().max()) < 2e-6
    res = check_forward(a, inp, tau, dtype, scale=scale)
    check_forward(b, inp, tau, dtype, scale=scale, ref=res["ref"] if res["nflip"] == 0 else None)


def test_rho_sweep_small():
    inp = make_inputs(2, 256, 2, 64, dtype="bf16", seed=30)
    e = oracle.forward(**inp, tau=np.full(2, INF, np.float32), scale=0.125)["e"]
    for rho in (0.0, 0.1, 0.25, 0.5, 1.0):
        tau = tau_for_rho(e, rho)
        out = _run(inp, tau, torch.bfloat16, scale=0.125)
        res = check_forward(out, inp, tau, torch.bfloat16, scale=0.125)
        want = 2 * int(round(rho * 2 * 256))          # round(rho*B*T) per head, 2 heads
        got = int(out["count"].sum())
        assert abs(got - want) <= res["nflip"], (rho, got, want)


@pytest.mark.parametrize("B,T,H,dk,dv", [
    (1, 63, 1, 128, 128), (1, 64, 2, 64, 64), (2, 65, 1, 64, 128), (1, 127, 2, 128, 64),
    (1, 128, 1, 128, 128), (2, 129, 3, 64, 64), (3, 150, 5, 128, 128), (1, 257, 7, 64, 128)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_chunk_boundaries(B, T, H, dk, dv, dtype):
    """Lengths on either side of the 64-token chunk and 64/128-query blocks (the
    token-serial path below 65 tokens, the chunked path above), several head counts."""
    seed = 40 + T + H
    inp = make_inputs(B, T, H, dk, dv, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    scale = dk ** -0.5
    tau = _tau(inp, 0.5, scale)
    out = _run(inp, tau, dtype, scale=scale)
    check_forward(out, inp, tau, dtype, scale=scale)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_decode_from_empty_state(dtype):
    """Decode steps from a zero state and an empty cache equal one forward call;
    with tau = +inf nothing is cached and o_kv stays 0."""
    B, H, d, T = 2, 3, 64, 20
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=33)
    scale = d ** -0.5
    for tau in (_tau(inp, 0.5, scale), np.full(H, INF, np.float32)):
        ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T)
        t = to_dev(inp, dtype, DEV)
        tau_d = torch.from_numpy(tau).to(DEV)
        S = torch.zeros((B, H, d, d), device=DEV)
        Kc = torch.zeros((B, H, T, d), dtype=dtype, device=DEV)
        Vc = torch.zeros((B, H, T, d), dtype=dtype, device=DEV)
        pos = torch.full((B, H, T), -1, dtype=torch.int32, device=DEV)
        count = torch.zeros((B, H), dtype=torch.int32, device=DEV)
        plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale, want_o_kv=True)
        es, rs, os_, okv = [], [], [], []
        for s in range(T):
            x = {n: t[n][:, s].contiguous() for n in t}
            plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, Kc, Vc, pos, count,
                 torch.full((B,), s, dtype=torch.int32, device=DEV))
            es.append(plan.e.cpu().numpy()); rs.append(plan.routed.cpu().numpy())
            os_.append(np_of(plan.o)); okv.append(np_of(plan.o_kv))
        torch.cuda.synchronize()
        e_all, r_all = np.stack(es, 1), np.stack(rs, 1)
        nflip = check_routing(e_all, r_all, ref, tau)
        if nflip:
            ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, mask_override=r_all)
        assert np.all(e_all[:, 0] == 1.0)               # zero state: cosine 0 by definition
        assert rel_err_slices(np.stack(os_, 1), ref["o"], 2) < TOL[dtype]
        assert np.array_equal(count.cpu().numpy(), ref["count"])
        if np.isinf(tau).all():
            assert int(count.sum()) == 0 and float(np.abs(np.stack(okv, 1)).max()) == 0.0
        else:
            assert rel_err_slices(np.stack(okv, 1), ref["o_kv"], 2) < TOL[dtype]
            got_pos = pos.cpu().numpy()
            for b in range(B):
                for h in range(H):
                    n = int(ref["count"][b, h])
                    assert np.array_equal(got_pos[b, h, :n], ref["pos"][b, h, :n])

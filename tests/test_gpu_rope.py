"""GPU parity of rotary position embedding on the attention path.

RoPE ("Hybrid Associative Memories", §5 model setup: base 500K on the attention
layers; RoFormer §3.4.2 for the rotation) turns the attention query and key of
each token by angles pos * base^(-2i/d) on consecutive element pairs, at the
token's absolute position.  The KV cache holds the rotated keys, so a key is
turned once, at the position where it was written.  Compared with the oracle
through the C ABI: routing as in the unrotated path (the RNN never sees the
rotation), pos and Vc exactly, Kc and the outputs within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, make_gates, tau_for_rho
from parity import check_forward, check_routing, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _tau(inp, rho, scale):
    e = oracle.forward(**inp, tau=np.full(inp["q"].shape[2], INF, np.float32), scale=scale)["e"]
    return tau_for_rho(e, rho)


def _dt(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


@pytest.mark.parametrize("B,T,H,dk,dv,base,t0,rec", [
    (2, 200, 3, 128, 128, 500000.0, 0, False),
    (1, 65, 2, 64, 128, 10000.0, 0, False),
    (2, 130, 2, 128, 64, 10000.0, 37, False),
    (1, 97, 2, 64, 64, 500000.0, 1000000, False),
    (2, 150, 2, 128, 128, 10000.0, 5, True),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_forward(B, T, H, dk, dv, base, t0, rec, dtype):
    seed = 90 + T + dk
    inp = make_inputs(B, T, H, dk, dv, dtype=_dt(dtype), seed=seed)
    scale = dk ** -0.5
    tau = _tau(inp, 0.5, scale)
    gr, gk = make_gates(B, T, H, seed)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, gate_rnn=torch.from_numpy(gr).to(DEV),
                          gate_kv=torch.from_numpy(gk).to(DEV), t0=t0, rope_base=base,
                          force_recurrent=rec, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    check_forward(out, inp, tau, dtype, scale=scale, gates=(gr, gk), t0=t0, rope_base=base)


def test_rope_changes_the_readout():
    """The rotation is applied: the attention readout with RoPE differs from the
    one without, while scores, routing and the RNN readout do not change."""
    B, T, H, d = 1, 130, 2, 64
    inp = make_inputs(B, T, H, d, dtype="f32", seed=95)
    tau = _tau(inp, 0.5, 0.125)
    t = to_dev(inp, torch.float32, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    kw = dict(scale=0.125, want_o_rnn=True, want_o_kv=True)
    a = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], tau_d, **kw)
    r = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], tau_d, rope_base=10000.0, **kw)
    torch.cuda.synchronize()
    assert torch.equal(a["e"], r["e"]) and torch.equal(a["routed"], r["routed"])
    assert torch.equal(a["o_rnn"], r["o_rnn"]) and torch.equal(a["Vc"], r["Vc"])
    assert (a["o_kv"] - r["o_kv"]).abs().max().item() > 1e-3


def test_rope_separate_attention_inputs():
    """With separate attention projections the rotation acts on q_attn and k_attn."""
    B, T, H, d = 1, 130, 2, 64
    inp = make_inputs(B, T, H, d, seed=96)
    att = make_inputs(B, T, H, d, seed=97)
    tau = _tau(inp, 0.4, 1.0)
    t = to_dev(inp, torch.float32, DEV)
    ta = to_dev(att, torch.float32, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=1.0, q_attn=ta["q"], k_attn=ta["k"], v_attn=ta["v"],
                          rope_base=500000.0, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    check_forward(out, inp, tau, torch.float32, scale=1.0, attn=att, rope_base=500000.0)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_continuation_equals_one_call(dtype):
    """Two calls (the second with t0 = length of the first and the first's cache)
    rotate every key at its own absolute position."""
    B, T, H, d = 2, 190, 2, 64
    base = 500000.0
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=98)
    scale = 0.125
    tau = _tau(inp, 0.5, scale)
    T1 = 77
    first = {n: a[:, :T1] for n, a in inp.items()}
    second = {n: a[:, T1:] for n, a in inp.items()}
    t1, t2 = to_dev(first, dtype, DEV), to_dev(second, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    o1 = ham.ham_forward(t1["q"], t1["k"], t1["v"], t1["beta"], t1["g"], tau_d, scale=scale, cap=T,
                         rope_base=base)
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    o2 = ham.ham_forward(t2["q"], t2["k"], t2["v"], t2["beta"], t2["g"], tau_d, scale=scale,
                         S0=o1["S"].clone(), cache=cache, t0=T1, rope_base=base,
                         want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    ref1 = oracle.forward(**first, tau=tau, scale=scale, cap=T, rope_base=base)
    ref_cache = {n: ref1[n] for n in ("Kc", "Vc", "pos", "count")}
    check_routing(o1["e"].cpu().numpy(), o1["routed"].cpu().numpy(), ref1, tau)
    check_forward(o2, second, tau, dtype, scale=scale, S0=ref1["S"], cache=ref_cache, t0=T1,
                  rope_base=base)
    # and the whole sequence in one oracle call gives the same second-half readout
    full = oracle.forward(**inp, tau=tau, scale=scale, cap=T, rope_base=base,
                          mask_override=np.concatenate([o1["routed"].cpu().numpy(),
                                                        o2["routed"].cpu().numpy()], 1))
    assert rel_err_slices(np_of(o2["o"]), full["o"][:, T1:], 2) < TOL[dtype]


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rope_decode_steps_equal_forward(dtype):
    B, H, d = 3, 2, 128
    T0, steps = 70, 24
    T = T0 + steps
    base = 500000.0
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=99)
    scale = d ** -0.5
    tau = _tau(inp, 0.5, scale)
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, rope_base=base)
    t = to_dev(inp, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    o1 = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d, scale=scale,
                         cap=T, rope_base=base)
    S = o1["S"]
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale, rope_base=base)
    es, rs, os_ = [], [], []
    for s in range(steps):
        tt = T0 + s
        x = {n: t[n][:, tt].contiguous() for n in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, cache["Kc"], cache["Vc"],
             cache["pos"], cache["count"], torch.full((B,), tt, dtype=torch.int32, device=DEV))
        es.append(plan.e.cpu().numpy()); rs.append(plan.routed.cpu().numpy())
        os_.append(np_of(plan.o))
    torch.cuda.synchronize()
    assert int(plan.status.item()) == 0
    e_all = np.concatenate([o1["e"].cpu().numpy(), np.stack(es, 1)], 1)
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rs, 1)], 1)
    if check_routing(e_all, r_all, ref, tau):
        ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, rope_base=base, mask_override=r_all)
    assert rel_err_slices(np.stack(os_, 1), ref["o"][:, T0:], 2) < TOL[dtype]
    cnt = cache["count"].cpu().numpy()
    assert np.array_equal(cnt, ref["count"])
    Kc = np_of(cache["Kc"])
    for b in range(B):
        for h in range(H):
            n = cnt[b, h]
            kr = ref["Kc"][b, h, :n]
            assert np.abs(Kc[b, h, :n] - kr).max() / np.abs(kr).max() < (1e-5 if dtype == torch.float32 else 8e-3)


def test_rope_decode_per_sequence_positions():
    """Decode from an empty cache with a different absolute position per sequence
    (t_abs[b] = start_b + step) matches the oracle run with per-sequence t0."""
    B, H, d, steps = 4, 2, 64, 12
    base = 10000.0
    start = np.array([0, 5, 4093, 123456], np.int64)
    inp = make_inputs(B, steps, H, d, dtype="f32", seed=100)
    scale = d ** -0.5
    tau = np.full(H, -INF, np.float32)             # route every token
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=steps, t0=start, rope_base=base)
    t = to_dev(inp, torch.float32, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device=DEV)
    Kc = torch.zeros((B, H, steps, d), dtype=torch.float32, device=DEV)
    Vc = torch.zeros_like(Kc)
    pos = torch.full((B, H, steps), -1, dtype=torch.int32, device=DEV)
    count = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    plan = ham.DecodePlan(B, H, d, d, steps, torch.float32, DEV, scale=scale, rope_base=base)
    outs = []
    for s in range(steps):
        x = {n: t[n][:, s].contiguous() for n in t}
        t_abs = torch.from_numpy((start + s).astype(np.int32)).to(DEV)
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, Kc, Vc, pos, count, t_abs)
        outs.append(np_of(plan.o))
    torch.cuda.synchronize()
    assert np.array_equal(pos.cpu().numpy(), ref["pos"])
    assert rel_err_slices(np_of(Kc), ref["Kc"], 1) < 1e-5
    assert rel_err_slices(np.stack(outs, 1), ref["o"], 2) < TOL[torch.float32]


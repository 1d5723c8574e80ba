"""GPU parity of the learned-router path and of the threshold selection.

A learned input router ("Hybrid Associative Memories", App. A.1 "Router
Implementations": sigma(W_r x_t), computed by the caller) supplies the routing
scores; the layer then routes by score > tau and the RNN still reads every token.
ham_select_tau sets the per-head threshold for a target KV fraction (§5 rho_KV).
Both run through the C ABI and are compared with the oracle: routing, cache and
threshold exactly, outputs within the dtype tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, make_gates, make_router_scores
from parity import check_forward, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _router_scores(B, T, H, seed):
    """Scores in (0, 1) like sigma(W_r x); a few are set exactly to the threshold
    afterwards by the tests (ties do not route)."""
    return make_router_scores(B, T, H, seed).copy()


@pytest.mark.parametrize("B,T,H,dk,dv", [(2, 200, 3, 128, 128), (1, 65, 2, 64, 128),
                                         (1, 40, 2, 64, 64), (2, 130, 2, 128, 64)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_scores_forward(B, T, H, dk, dv, dtype):
    seed = 60 + T + dk
    inp = make_inputs(B, T, H, dk, dv, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    rs = _router_scores(B, T, H, seed)
    tau = oracle.select_tau(rs, 0.4)
    rs[0, :3, 0] = tau[0]                                   # exact ties never route
    gr, gk = make_gates(B, T, H, seed)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=dk ** -0.5, gate_rnn=torch.from_numpy(gr).to(DEV),
                          gate_kv=torch.from_numpy(gk).to(DEV), router_scores=torch.from_numpy(rs).to(DEV),
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    assert int(out["routed"][0, :3, 0].sum()) == 0
    check_forward(out, inp, tau, dtype, scale=dk ** -0.5, gates=(gr, gk), router_score=rs)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_decode_steps_equal_forward(dtype):
    B, H, d = 2, 3, 64
    T0, steps = 70, 16
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=71)
    rs = _router_scores(B, T, H, 71)
    tau = oracle.select_tau(rs, 0.5)
    scale = d ** -0.5
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, router_score=rs)
    t = to_dev(inp, dtype, DEV)
    rsd = torch.from_numpy(rs).to(DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
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
    r_all = np.concatenate([o1["routed"].cpu().numpy(), np.stack(rts, 1)], 1)
    assert np.array_equal(r_all.astype(bool), ref["routed"].astype(bool))
    assert np.array_equal(cache["count"].cpu().numpy(), ref["count"])
    assert rel_err_slices(np.stack(outs, 1), ref["o"][:, T0:], 2) < TOL[dtype]
    assert rel_err_slices(np_of(S), ref["S"], 1) < 1e-4


def _select_cases():
    rng = np.random.default_rng(80)
    cases = []
    cases.append(("normal", rng.standard_normal((2, 300, 3)).astype(np.float32)))
    q = np.round(rng.random((3, 257, 2)) * 8) / 8                      # many ties
    cases.append(("ties", q.astype(np.float32)))
    x = rng.standard_normal((1, 500, 4)).astype(np.float32)
    x[0, ::37, 1] = np.nan
    x[0, ::41, 2] = np.inf
    x[0, 3::43, 2] = -np.inf
    x[0, ::5, 3] = -0.0
    x[0, 1::5, 3] = 0.0
    cases.append(("nan_inf_zeros", x))
    cases.append(("pair", np.array([[[1.0], [2.0]]], np.float32)))
    cases.append(("layer_shape", rng.random((8, 4096, 16)).astype(np.float32) * 2.0))
    cases.append(("above_lds_staging", rng.standard_normal((2, 20011, 3)).astype(np.float32)))
    return cases


@pytest.mark.parametrize("name,e", _select_cases(), ids=[c[0] for c in _select_cases()])
def test_select_tau_matches_oracle(name, e):
    ed = torch.from_numpy(e).to(DEV)
    for rho in (0.0, 0.001, 0.1, 0.25, 0.5, 0.75, 0.9, 0.999, 1.0):
        got = ham.ham_select_tau(ed, rho).cpu().numpy()
        want = oracle.select_tau(e, rho)
        same = (got == want) | (np.isnan(got) & np.isnan(want))
        assert same.all(), (name, rho, got, want)


def test_select_tau_then_route_hits_the_fraction():
    """Thresholds chosen on the GPU for the fit-error scores route round(rho*B*T) tokens
    of every head when the scores are distinct."""
    B, T, H, d = 2, 256, 4, 64
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=81)
    t = to_dev(inp, torch.bfloat16, DEV)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], torch.full((H,), float("inf"), device=DEV),
                             want_rho=False)
    for rho in (0.1, 0.5, 0.9):
        tau = ham.ham_select_tau(st["e"], rho)
        st2 = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], tau, want_rho=False)
        e = st["e"].cpu().numpy()
        k = int(round(rho * B * T))
        for h in range(H):
            if len(np.unique(e[:, :, h])) == B * T:
                assert int(st2["count"][:, h].sum()) == k


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_router_one_routed_set_per_layer(dtype):
    """A learned router gives one score per token (sigma(W_r x_t) has no head index);
    broadcast over the heads with one threshold, every head routes the same tokens:
    the layer keeps one routed set (the per-layer T_KV of the memory accounting,
    App. E.4), each head caching its own k and v of those tokens."""
    B, T, H, d = 2, 230, 4, 64
    inp = make_inputs(B, T, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=72)
    one = make_router_scores(B, T, 1, 72)
    rs = np.ascontiguousarray(np.broadcast_to(one, (B, T, H)))
    tau1 = oracle.select_tau(one, 0.3)
    tau = np.full(H, tau1[0], np.float32)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=d ** -0.5, router_scores=torch.from_numpy(rs).to(DEV),
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    r = out["routed"].cpu().numpy().astype(bool)
    assert (r == r[:, :, :1]).all()
    cnt = out["count"].cpu().numpy()
    assert (cnt == cnt[:, :1]).all() and int(cnt[0, 0]) == int((one[0, :, 0] > tau1[0]).sum())
    pos = out["pos"].cpu().numpy()
    for b in range(B):
        assert (pos[b, :, :cnt[b, 0]] == pos[b, :1, :cnt[b, 0]]).all()
    check_forward(out, inp, tau, dtype, scale=d ** -0.5, router_score=rs)


@pytest.mark.parametrize("B,T,H,dk,dv,kv", [(2, 200, 3, 128, 128, None), (1, 130, 2, 64, 128, None),
                                            (2, 150, 2, 128, 128, (4, 128, 64)),
                                            (1, 257, 2, 256, 384, (4, 128, 192))])
def test_router_overlap_forward(B, T, H, dk, dv, kv):
    """HAM_OVERLAP: with learned-router scores the RNN runs on the library's second
    stream beside routing, compaction and attention, joined before the mix.  Routing,
    cache and state against the oracle exactly / at 1e-4, outputs at the bf16
    tolerance, and the same results as the serial learned-router path up to the
    rounding of the separate mix pass."""
    seed = 90 + T + dk
    inp = make_inputs(B, T, H, dk, dv, dtype="bf16", seed=seed)
    rs = _router_scores(B, T, H, seed)
    tau = oracle.select_tau(rs, 0.5)
    gr, gk = make_gates(B, T, H, seed)
    att = None
    kw = {}
    if kv is not None:
        Hk, dkk, dvk = kv
        att = make_inputs(B, T, Hk, dkk, dvk, dtype="bf16", seed=seed + 1)
        ta = to_dev(att, torch.bfloat16, DEV)
        kw = dict(q_attn=ta["q"], k_attn=ta["k"], v_attn=ta["v"])
        gk = np.random.default_rng(seed).random((B, T, Hk)).astype(np.float32)
    scale = (kv[1] if kv else dk) ** -0.5
    t = to_dev(inp, torch.bfloat16, DEV)
    args = (t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV))
    common = dict(scale=scale, gate_rnn=torch.from_numpy(gr).to(DEV), gate_kv=torch.from_numpy(gk).to(DEV),
                  router_scores=torch.from_numpy(rs).to(DEV), want_o_rnn=True, want_o_kv=True, **kw)
    print(f"overlap: B={B} T={T} H={H} {dk}/{dv} kv={kv}", flush=True)
    ovl = ham.ham_forward(*args, overlap=True, **common)
    ser = ham.ham_forward(*args, overlap=False, **common)
    torch.cuda.synchronize()
    check_forward(ovl, inp, tau, torch.bfloat16, scale=scale, gates=(gr, gk), router_score=rs, attn=att)
    for n in ("routed", "count", "pos", "Kc", "Vc"):
        assert torch.equal(ovl[n], ser[n]), n
    assert torch.equal(ovl["S"], ser["S"])
    assert rel_err_slices(np_of(ovl["o"]), np_of(ser["o"]), 2) < 1e-2


def test_router_overlap_calls_in_a_row():
    """Overlapped calls back to back on one stream, on two shapes, each against the
    serial path (the second stream and its events are reused)."""
    outs = []
    for (B, T, H, d, seed) in ((2, 300, 2, 128, 95), (1, 100, 3, 64, 96), (2, 300, 2, 128, 97)):
        inp = make_inputs(B, T, H, d, dtype="bf16", seed=seed)
        rs = _router_scores(B, T, H, seed)
        tau = torch.from_numpy(oracle.select_tau(rs, 0.3)).to(DEV)
        t = to_dev(inp, torch.bfloat16, DEV)
        r = torch.from_numpy(rs).to(DEV)
        a = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, router_scores=r, overlap=True)
        b = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], tau, router_scores=r, overlap=False)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert torch.equal(a["S"], b["S"]) and torch.equal(a["count"], b["count"])
        assert rel_err_slices(np_of(a["o"]), np_of(b["o"]), 2) < 1e-2

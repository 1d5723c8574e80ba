"""GPU parity of block-contiguous routing.

"Hybrid Associative Memories" §7 (compute and memory performance): per-token
routing makes the KV cache a random gather from the residual stream; the pages
propose routing contiguous blocks of tokens instead and give no rule for it.  The
reading built here: positions are cut into aligned blocks of n tokens; a block
routes whole when the mean of its tokens' scores exceeds tau (at the block's last
token), and it enters the cache at that token, so queries see a routed block from
its last token on.  A forward call covers whole blocks; decode steps keep the open
block in cache rows past count and commit it at its last token.  Compared with the
oracle through the C ABI: routing per block except blocks whose mean lies within
1e-5 of tau, compaction exactly, outputs within tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import (make_inputs, make_gates, make_doc_start,
                                                  make_router_scores, tau_for_rho)
from parity import (check_forward, check_routing, np_of, rel_err_slices, to_dev, TOL, block_means,
                    spread_block_flags)

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _dt(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


def _i32(x):
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.int32))).to(DEV)


def _tau_blocks(inp, n, rho, scale, t0=0):
    """Per-head tau that routes about rho of the complete blocks (on block means)."""
    H = inp["q"].shape[2]
    e = oracle.forward(**inp, tau=np.full(H, INF, np.float32), scale=scale, t0=t0)["e"]
    T = e.shape[1]
    nb = T // n
    means = block_means(e, n)[:, :nb * n:n]
    return tau_for_rho(means, rho)


@pytest.mark.parametrize("B,T,H,dk,dv,n,rec,base,t0", [
    (2, 256, 3, 128, 128, 16, False, 0.0, 0),
    (1, 320, 2, 64, 128, 64, False, 500000.0, 64),
    (2, 192, 2, 128, 64, 4, True, 0.0, 0),
    (1, 96, 2, 64, 64, 32, False, 10000.0, 32),
    (2, 130, 2, 128, 128, 2, False, 0.0, 6),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_forward(B, T, H, dk, dv, n, rec, base, t0, dtype):
    seed = 140 + T + n
    inp = make_inputs(B, T, H, dk, dv, dtype=_dt(dtype), seed=seed)
    scale = dk ** -0.5
    tau = _tau_blocks(inp, n, 0.5, scale, t0)
    gr, gk = make_gates(B, T, H, seed)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, gate_rnn=torch.from_numpy(gr).to(DEV),
                          gate_kv=torch.from_numpy(gk).to(DEV), t0=t0, rope_base=base,
                          force_recurrent=rec, route_block=n, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    res = check_forward(out, inp, tau, dtype, scale=scale, gates=(gr, gk), t0=t0, rope_base=base,
                        route_block=n)
    r = out["routed"].cpu().numpy()
    assert np.array_equal(r, np.repeat(r[:, n - 1::n], n, axis=1))       # whole blocks
    assert 0 < r.mean() < 1
    assert res["ref"]["count"].min() % n == 0


@pytest.mark.parametrize("n", [8, 64])
def test_block_learned_router(n):
    """Learned-router scores: the block mean of the caller's scores decides."""
    B, T, H, d = 2, 256, 2, 64
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=150)
    rs = make_router_scores(B, T, H, 150)
    nb = T // n
    tau = tau_for_rho(rs.reshape(B, nb, n, H).astype(np.float64).mean(axis=2), 0.4)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=0.125, router_scores=torch.from_numpy(rs).to(DEV), route_block=n,
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    check_forward(out, inp, tau, torch.bfloat16, scale=0.125, router_score=rs, route_block=n)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_doc_mask_and_schedule(dtype):
    """Documents that start inside a block, and a threshold schedule along the
    sequence (tau taken at each block's last token)."""
    B, T, H, d, n = 2, 384, 2, 128, 16
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=151)
    ds = make_doc_start(B, T, 37, 151)
    scale = d ** -0.5
    base = _tau_blocks(inp, n, 0.5, scale)
    ramp = np.linspace(-0.05, 0.05, T, dtype=np.float32)
    tau = np.ascontiguousarray((base[None, None, :] + ramp[None, :, None]).repeat(B, 0)).astype(np.float32)
    t = to_dev(inp, dtype, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, doc_start=_i32(ds), rope_base=500000.0, route_block=n,
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    check_forward(out, inp, tau, dtype, scale=scale, doc_start=ds, rope_base=500000.0, route_block=n)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_continuation_equals_one_call(dtype):
    B, T, H, d, n = 2, 320, 2, 64, 32
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=152)
    scale = 0.125
    tau = _tau_blocks(inp, n, 0.5, scale)
    T1 = 128
    first = {k: a[:, :T1] for k, a in inp.items()}
    second = {k: a[:, T1:] for k, a in inp.items()}
    t1, t2 = to_dev(first, dtype, DEV), to_dev(second, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    o1 = ham.ham_forward(t1["q"], t1["k"], t1["v"], t1["beta"], t1["g"], tau_d, scale=scale, cap=T,
                         route_block=n)
    cache = {k: o1[k] for k in ("Kc", "Vc", "pos", "count")}
    o2 = ham.ham_forward(t2["q"], t2["k"], t2["v"], t2["beta"], t2["g"], tau_d, scale=scale,
                         S0=o1["S"].clone(), cache=cache, t0=T1, route_block=n,
                         want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    ref1 = oracle.forward(**first, tau=tau, scale=scale, cap=T, route_block=n)
    check_routing(o1["e"].cpu().numpy(), o1["routed"].cpu().numpy(), ref1, tau, n)
    r_all = np.concatenate([o1["routed"].cpu().numpy(), o2["routed"].cpu().numpy()], 1)
    full = oracle.forward(**inp, tau=tau, scale=scale, cap=T, route_block=n, mask_override=r_all)
    assert np.array_equal(o2["count"].cpu().numpy(), full["count"])
    assert rel_err_slices(np_of(o2["o"]), full["o"][:, T1:], 2) < TOL[dtype]


@pytest.mark.parametrize("n,base,docs", [(8, 0.0, False), (16, 500000.0, True), (4, 10000.0, False)])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_block_decode_steps_equal_forward(n, base, docs, dtype):
    """A forward prefix of whole blocks, then decode steps over several blocks (the
    last one left open): every step's output, the final cache and the routing equal
    one oracle forward over the whole sequence."""
    B, H, d = 3, 2, 128
    T0 = 8 * n
    steps = 2 * n + n // 2 + 1
    T = T0 + steps
    inp = make_inputs(B, T, H, d, dtype=_dt(dtype), seed=153 + n)
    scale = d ** -0.5
    tau = _tau_blocks(inp, n, 0.5, scale)
    ds = make_doc_start(B, T, 3 * n, 153) if docs else None
    t = to_dev(inp, dtype, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    pre = {k: x[:, :T0].contiguous() for k, x in t.items()}
    o1 = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d, scale=scale,
                         cap=T, rope_base=base, route_block=n,
                         doc_start=_i32(ds[:, :T0]) if docs else None)
    S = o1["S"]
    cache = {k: o1[k] for k in ("Kc", "Vc", "pos", "count")}
    plan = ham.DecodePlan(B, H, d, d, T, dtype, DEV, scale=scale, rope_base=base, route_block=n)
    es, rs, os_ = [], [], []
    for s in range(steps):
        tt = T0 + s
        x = {k: t[k][:, tt].contiguous() for k in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, S, cache["Kc"], cache["Vc"],
             cache["pos"], cache["count"], torch.full((B,), tt, dtype=torch.int32, device=DEV),
             doc_start=_i32(ds[:, tt]) if docs else None)
        es.append(plan.e.cpu().numpy()); rs.append(plan.routed.cpu().numpy())
        os_.append(np_of(plan.o))
    torch.cuda.synchronize()
    assert int(plan.status.item()) == 0
    e_all = np.concatenate([o1["e"].cpu().numpy(), np.stack(es, 1)], 1)
    r_dec = np.stack(rs, 1)
    assert not r_dec[:, [s for s in range(steps) if (T0 + s) % n != n - 1]].any()
    r_all = np.concatenate([o1["routed"].cpu().numpy(), spread_block_flags(r_dec, n)], 1)
    okw = dict(tau=tau, scale=scale, cap=T, rope_base=base, route_block=n, doc_start=ds)
    ref = oracle.forward(**inp, **okw)
    if check_routing(e_all, r_all, ref, tau, n):
        ref = oracle.forward(**inp, mask_override=r_all, **okw)
    assert np.array_equal(r_all.astype(bool), ref["routed"].astype(bool))
    assert rel_err_slices(np.stack(os_, 1), ref["o"][:, T0:], 2) < TOL[dtype]
    cnt = cache["count"].cpu().numpy()
    assert np.array_equal(cnt, ref["count"])
    pos = cache["pos"].cpu().numpy()
    Vc = np_of(cache["Vc"])
    for b in range(B):
        for h in range(H):
            c = cnt[b, h]
            assert np.array_equal(pos[b, h, :c], ref["pos"][b, h, :c])
            assert np.array_equal(Vc[b, h, :c], ref["Vc"][b, h, :c])
    # the open block's score sum, carried for the next step
    j = T % n
    want = e_all[:, T - j:].astype(np.float64).sum(axis=1)
    assert np.abs(plan.block_score.cpu().numpy() - want).max() < 1e-4


def test_block_route_stats():
    B, T, H, d, n = 2, 512, 4, 128, 16
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=154)
    tau = _tau_blocks(inp, n, 0.25, 1.0)
    t = to_dev(inp, torch.bfloat16, DEV)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                             route_block=n)
    ref = oracle.forward(**inp, tau=tau, scale=1.0, route_block=n)
    nflip = check_routing(st["e"].cpu().numpy(), st["routed"].cpu().numpy(), ref, tau, n)
    cnt = st["count"].cpu().numpy()
    assert np.abs(cnt - ref["count"]).sum() <= n * nflip
    assert np.array_equal(cnt, st["routed"].cpu().numpy().astype(np.int64).sum(axis=1))
    assert st["n_near"] is None and abs(st["rho"] - cnt.sum() / (B * T * H)) < 1e-12


def test_block_decode_capacity():
    """Rows of an open block that would land past cap are dropped and flagged; the
    count never exceeds cap."""
    B, H, d, n = 2, 2, 64, 8
    cap = 12
    inp = make_inputs(B, 2 * n, H, d, dtype="f32", seed=155)
    t = to_dev(inp, torch.float32, DEV)
    tau = torch.full((H,), -float("inf"), device=DEV)
    S = torch.zeros((B, H, d, d), device=DEV)
    Kc = torch.zeros((B, H, cap, d), device=DEV)
    Vc = torch.zeros_like(Kc)
    pos = torch.full((B, H, cap), -1, dtype=torch.int32, device=DEV)
    count = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    plan = ham.DecodePlan(B, H, d, d, cap, torch.float32, DEV, route_block=n)
    for s in range(2 * n):
        x = {k: t[k][:, s].contiguous() for k in t}
        plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau, S, Kc, Vc, pos, count,
             torch.full((B,), s, dtype=torch.int32, device=DEV))
        torch.cuda.synchronize()
        c = count.cpu().numpy()
        assert (c <= cap).all()
        if s == n - 1:
            assert (c == n).all() and int(plan.status.item()) == 0
    assert int(plan.status.item()) == 1
    assert (count.cpu().numpy() == cap).all()
    assert np.array_equal(pos.cpu().numpy()[:, :, :n], np.broadcast_to(np.arange(n), (B, H, n)))

"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times, against the CPU oracle on everything it can afford: every routing score,
routing decision, compaction entry and final state of every head (RNN-only oracle
pass), and the attention outputs at sampled tokens of sampled heads -- at the
headline layer at rho = 0.5, every output element of every head.

Workloads: the layer at the 800M-model shape (B=8, H=16, d=128, T=4096, bf16 I/O,
rho = 0.5, the two rho limits and the sweep's 0.1 and 0.25; rho = 0.5 with RoPE base 500K; rho = 0.5 over packed
documents with same-document masking and RoPE; rho = 0.5 of 64-token blocks with
block-contiguous routing; 32 KV heads of 128/64, and the 800M layer's 5 RNN heads of 256/384 with
10 KV heads of 128/192, at sampled sequence-head pairs); the long-context case (B=1, H=16, T=32768,
planted repeated pairs, rho = 0.25); the decode case (batch 32, H=16, d=128,
32K-token prefix, then 16 decode steps, 64 sampled sequence-head pairs).
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import (LAYER, LONG, DECODE_B, DECODE_D, DECODE_H,
                                                  DECODE_PREFIX, make_doc_start, make_inputs,
                                                  make_inputs_torch, make_router_scores,
                                                  make_workload, tau_for_rho)
from parity import E_TOL, NEAR, TOL, block_means, np_of, rel_err_slices, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _rnn_only_oracle(inp, tau, scale, cap=None, rope_base=0.0, route_block=0):
    """Oracle over all heads with no attention readout (emit all-zero)."""
    B, T, H, _ = inp["q"].shape
    return oracle.forward(**inp, tau=tau, scale=scale, cap=cap, emit=np.zeros((B, T, H), np.int8),
                          rope_base=rope_base, route_block=route_block)


def _check_all_heads(out, ref, tau, kc_tol=None, route_block=0):
    """Scores, routing, compaction and state of every head.  kc_tol: None for
    bit-exact cached keys, else the per-slice relative tolerance (rotated keys).
    route_block > 1: the near band applies to block means."""
    e_gpu = out["e"].cpu().numpy()
    r_gpu = out["routed"].cpu().numpy().astype(bool)
    de = np.abs(e_gpu - ref["e"]).max()
    assert de < E_TOL, f"score error {de:.3e}"
    H = e_gpu.shape[2]
    score = ref["e"] if route_block <= 1 else block_means(ref["e"], route_block)
    near = np.abs(score - np.asarray(tau, np.float64).reshape(1, 1, H)) < NEAR
    flips = r_gpu != ref["routed"].astype(bool)
    assert not (flips & ~near).any(), f"{int((flips & ~near).sum())} flips outside the near band"
    nflip_heads = flips.any(axis=1)                      # [B,H]
    cnt = out["count"].cpu().numpy()
    pos = out["pos"].cpu().numpy()
    Kc, Vc = out["Kc"], out["Vc"]
    B = cnt.shape[0]
    for b in range(B):
        for h in range(H):
            if nflip_heads[b, h]:
                # routing differs only inside the band: compaction must be the GPU mask's nonzeros
                nz = np.nonzero(r_gpu[b, :, h])[0]
                assert cnt[b, h] == len(nz)
                assert np.array_equal(pos[b, h, :len(nz)], nz)
                continue
            n = int(ref["count"][b, h])
            assert cnt[b, h] == n
            assert np.array_equal(pos[b, h, :n], ref["pos"][b, h, :n])
            if kc_tol is None:
                assert np.array_equal(np_of(Kc[b, h, :n]), ref["Kc"][b, h, :n])
            elif n:
                kr = ref["Kc"][b, h, :n]
                assert np.abs(np_of(Kc[b, h, :n]) - kr).max() / np.abs(kr).max() < kc_tol
            assert np.array_equal(np_of(Vc[b, h, :n]), ref["Vc"][b, h, :n])
    errS = rel_err_slices(np_of(out["S"]), ref["S"], 1)
    assert errS < 1e-4, errS
    return int(flips.sum()), float(de)


def _check_sampled_outputs(out, inp, tau, scale, heads, ntok, dtype, seed, r_gpu, rope_base=0.0,
                           doc_start=None, route_block=0):
    """Oracle outputs at sampled tokens of sampled heads (with the GPU mask if it
    differs from the oracle's inside the near band)."""
    T = inp["q"].shape[1]
    rng = np.random.default_rng(seed)
    worst = {}
    for (b, h) in heads:
        sub = {n: np.ascontiguousarray(a[b:b + 1, :, h:h + 1]) for n, a in inp.items()}
        toks = np.unique(np.concatenate([rng.choice(T, ntok, replace=False), [0, T - 1]]))
        emit = np.zeros((1, T, 1), np.int8)
        emit[0, toks, 0] = 1
        ref = oracle.forward(**sub, tau=tau[h:h + 1], scale=scale, emit=emit,
                             mask_override=r_gpu[b:b + 1, :, h:h + 1], rope_base=rope_base,
                             doc_start=None if doc_start is None else doc_start[b:b + 1],
                             route_block=route_block)
        for name in ("o", "o_rnn", "o_kv"):
            x = np_of(out[name][b, toks, h])
            y = ref[name][0, toks, 0]
            err = np.abs(x - y).max() / max(np.abs(y).max(), 1e-30)
            worst[name] = max(worst.get(name, 0.0), float(err))
            assert err < TOL[dtype], (name, b, h, err)
    return worst


@pytest.mark.parametrize("rho", [0.5, 0.0, 1.0, 0.1, 0.25])
def test_layer_fullsize(rho):
    w = LAYER
    inp = make_workload(w)
    scale = w.attn_scale
    tau0 = np.full(w.H, INF, np.float32)
    base = _rnn_only_oracle(inp, tau0, scale)
    tau = tau_for_rho(base["e"], rho)
    ref = _rnn_only_oracle(inp, tau, scale)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref, tau)
    r_gpu = out["routed"].cpu().numpy()
    # each head's threshold routes round(rho * B * T) of its tokens (up to near-band flips)
    want = w.H * round(rho * w.B * w.T)
    assert abs(int(out["count"].sum()) - want) <= nflip + 1, (int(out["count"].sum()), want, nflip)
    worst = _check_sampled_outputs(out, inp, tau, scale, [(0, 0), (3, 7), (7, 15)], 24,
                                   torch.bfloat16, 40, r_gpu)
    print(f"layer rho={rho}: max|de|={de:.2e} near-band flips={nflip} sampled errors {worst}")


def test_layer_fullsize_every_output():
    """The headline layer (B=8, H=16, T=4096, d=128, bf16, rho = 0.5) with every
    output element compared: the oracle's full forward (all heads, all tokens) runs
    with the GPU's routing mask, so near-threshold flips do not matter, and o, o_rnn
    and o_kv of every (b, h) slice must meet the bf16 tolerance; the scores, cache
    and state are checked for every head as above."""
    w = LAYER
    inp = make_workload(w)
    scale = w.attn_scale
    base = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base["e"], 0.5)
    ref_rnn = _rnn_only_oracle(inp, tau, scale)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref_rnn, tau)
    r_gpu = out["routed"].cpu().numpy()
    ref = oracle.forward(**inp, tau=tau, scale=scale, mask_override=r_gpu)
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"layer, every output: max|de|={de:.2e} near-band flips={nflip} worst slice errors {worst}")


def test_layer_fullsize_rope():
    """The layer at rho = 0.5 with RoPE base 500K on the attention path."""
    w = LAYER
    base = 500000.0
    inp = make_workload(w)
    scale = w.attn_scale
    base_e = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base_e["e"], 0.5)
    ref = _rnn_only_oracle(inp, tau, scale, rope_base=base)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, rope_base=base, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref, tau, kc_tol=8e-3)
    worst = _check_sampled_outputs(out, inp, tau, scale, [(0, 0), (4, 9), (7, 15)], 24,
                                   torch.bfloat16, 42, out["routed"].cpu().numpy(), rope_base=base)
    print(f"layer rope: max|de|={de:.2e} near-band flips={nflip} sampled errors {worst}")


def test_layer_fullsize_packed_documents():
    """The layer at rho = 0.5 over packed batches (geometric document lengths, mean
    1024 tokens) with same-document masking and RoPE base 500K."""
    w = LAYER
    inp = make_workload(w)
    scale = w.attn_scale
    ds = make_doc_start(w.B, w.T, 1024, 43)
    base_e = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base_e["e"], 0.5)
    ref = _rnn_only_oracle(inp, tau, scale, rope_base=500000.0)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, rope_base=500000.0,
                          doc_start=torch.from_numpy(ds.astype(np.int32)).to(DEV),
                          want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref, tau, kc_tol=8e-3)
    worst = _check_sampled_outputs(out, inp, tau, scale, [(0, 1), (2, 8), (6, 14)], 32,
                                   torch.bfloat16, 44, out["routed"].cpu().numpy(),
                                   rope_base=500000.0, doc_start=ds)
    print(f"layer packed: max|de|={de:.2e} near-band flips={nflip} sampled errors {worst}")


def test_layer_fullsize_block_routing():
    """The layer with 64-token block-contiguous routing, tau per head for half of the
    blocks on their mean score (the benchmark's block-routing leg)."""
    w = LAYER
    n = 64
    inp = make_workload(w)
    scale = w.attn_scale
    base_e = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(block_means(base_e["e"], n)[:, ::n], 0.5)
    ref = _rnn_only_oracle(inp, tau, scale, route_block=n)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, route_block=n, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref, tau, route_block=n)
    r_gpu = out["routed"].cpu().numpy()
    assert np.array_equal(r_gpu, np.repeat(r_gpu[:, n - 1::n], n, axis=1))
    got_rho = float(out["count"].sum()) / (w.B * w.T * w.H)
    assert abs(got_rho - 0.5) <= (nflip + n) / (w.B * w.T * w.H)
    worst = _check_sampled_outputs(out, inp, tau, scale, [(0, 2), (5, 11), (7, 15)], 24,
                                   torch.bfloat16, 45, r_gpu, route_block=n)
    print(f"layer blocks: max|de|={de:.2e} near-band flips={nflip} sampled errors {worst}")


def test_long_context_fullsize():
    w = LONG
    inp = make_workload(w)
    scale = w.attn_scale
    base = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base["e"], w.rho)
    ref = _rnn_only_oracle(inp, tau, scale)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    nflip, de = _check_all_heads(out, ref, tau)
    worst = _check_sampled_outputs(out, inp, tau, scale, [(0, 0), (0, 9)], 16, torch.bfloat16, 41,
                                   out["routed"].cpu().numpy())
    print(f"long: max|de|={de:.2e} near-band flips={nflip} sampled errors {worst}")


@pytest.mark.parametrize("rho", [0.1, 1.0])
def test_layer_rho_every_output(rho):
    """The headline layer at the rho sweep's sparse and full ends (rho = 0.1, and 1.0:
    every token cached, full causal attention beside the RNN) with every output element
    of every head compared against the oracle's forward under the GPU's routing mask."""
    w = LAYER
    inp = make_workload(w)
    scale = w.attn_scale
    base = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base["e"], rho)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    r_gpu = out["routed"].cpu().numpy()
    if rho == 1.0:
        assert r_gpu.all()
    ref = oracle.forward(**inp, tau=tau, scale=scale, mask_override=r_gpu)
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"layer rho={rho}, every output: worst slice errors {worst}")


@pytest.mark.parametrize("overlap", [False, True])
def test_learned_router_every_output(overlap):
    """The headline layer with a learned router's scores (synthetic sigmoid scores, one
    per token and head) as the routing score, thresholds for rho = 0.5: the score-free
    state pass, alone or beside the attention chain on a second stream.  Routing must
    equal score > tau exactly, and every output element of every head must meet the bf16
    tolerance against the oracle."""
    w = LAYER
    inp = make_workload(w)
    scale = w.attn_scale
    rs = make_router_scores(w.B, w.T, w.H, 77).copy()
    tau = oracle.select_tau(rs, 0.5)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, router_scores=torch.from_numpy(rs).to(DEV), want_o_rnn=True,
                          want_o_kv=True, overlap=overlap)
    torch.cuda.synchronize()
    r_gpu = out["routed"].cpu().numpy().astype(bool)
    assert np.array_equal(r_gpu, rs > tau.reshape(1, 1, w.H))
    ref = oracle.forward(**inp, tau=tau, scale=scale, router_score=rs)
    assert np.array_equal(out["count"].cpu().numpy(), ref["count"])
    assert rel_err_slices(np_of(out["S"]), ref["S"], 1) < 1e-4
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"learned router (overlap={overlap}), every output: worst slice errors {worst}")


@pytest.mark.parametrize("variant", ["rope", "packed", "blocks", "kv32"])
def test_layer_variants_every_output(variant):
    """The benchmark's layer variants at full size (B 8, H 16, T 4096, bf16) with every
    output element compared: RoPE base 500K; packed documents (mean 1024) with RoPE;
    64-token block routing; 32 KV heads of 128/64 over the 16 RNN heads (the split-head
    mix).  The oracle's full forward runs with the GPU's routing mask; o, o_rnn and o_kv
    of every head must meet the bf16 tolerance."""
    w = LAYER
    scale = w.attn_scale
    kw, okw = {}, {}
    if variant == "kv32":
        inp = make_inputs(w.B, w.T, w.H, 128, 128, dtype="bf16", seed=188)
        att = make_inputs(w.B, w.T, 2 * w.H, 128, 64, dtype="bf16", seed=189)
        tau = np.full(w.H, 1.0, np.float32)
        ta = to_dev(att, torch.bfloat16, DEV)
        kw = dict(q_attn=ta["q"], k_attn=ta["k"], v_attn=ta["v"])
        okw = dict(q_attn=att["q"], k_attn=att["k"], v_attn=att["v"])
    else:
        inp = make_workload(w)
        base_e = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
        if variant == "blocks":
            tau = tau_for_rho(block_means(base_e["e"], 64)[:, ::64], 0.5)
            kw = okw = dict(route_block=64)
        else:
            tau = tau_for_rho(base_e["e"], 0.5)
            kw = dict(rope_base=500000.0)
            okw = dict(rope_base=500000.0)
            if variant == "packed":
                ds = make_doc_start(w.B, w.T, 1024, 43)
                kw["doc_start"] = torch.from_numpy(ds.astype(np.int32)).to(DEV)
                okw["doc_start"] = ds
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True, **kw)
    torch.cuda.synchronize()
    r_gpu = out["routed"].cpu().numpy()
    ref = oracle.forward(**inp, tau=tau, scale=scale, mask_override=r_gpu, **okw)
    de = np.abs(out["e"].cpu().numpy() - ref["e"]).max()
    assert de < E_TOL, de
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"layer {variant}, every output: max|de|={de:.2e} worst slice errors {worst}")


def test_long_context_every_output():
    """The long-context case (B=1, H=16, T=32768, rho = 0.25, the segmented state pass)
    with every output element compared: the oracle's full forward runs with the GPU's
    routing mask, and o, o_rnn and o_kv of every head must meet the bf16 tolerance."""
    w = LONG
    inp = make_workload(w)
    scale = w.attn_scale
    base = _rnn_only_oracle(inp, np.full(w.H, INF, np.float32), scale)
    tau = tau_for_rho(base["e"], w.rho)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    r_gpu = out["routed"].cpu().numpy()
    ref = oracle.forward(**inp, tau=tau, scale=scale, mask_override=r_gpu)
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"long, every output: worst slice errors {worst}")


def test_paper_heads_every_output():
    """The 800M layer's head geometry at full size (B 8, T 4096, bf16: 5 RNN heads of
    256/384 on the chunked state pass, 10 KV heads of 128/192 on the tiled attention):
    every score and final state of all 40 RNN heads, routing outside the near band, and
    every output element of o, o_rnn (per RNN head) and o_kv (per KV head) against the
    oracle's forward under the GPU's routing mask."""
    B, T, H, dk, dv, r, dkk = 8, 4096, 5, 256, 384, 2, 128
    inp = make_inputs(B, T, H, dk, dv, dtype="bf16", seed=60 + dk)
    att = make_inputs(B, T, r * H, dkk, dv // r, dtype="bf16", seed=61 + dk)
    tau = np.full(H, 1.0, np.float32)
    scale = dkk ** -0.5
    t, ta = to_dev(inp, torch.bfloat16, DEV), to_dev(att, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, q_attn=ta["q"], k_attn=ta["k"], v_attn=ta["v"], want_o_rnn=True,
                          want_o_kv=True)
    torch.cuda.synchronize()
    r_gpu = out["routed"].cpu().numpy()
    okw = dict(tau=tau, scale=scale, q_attn=att["q"], k_attn=att["k"], v_attn=att["v"])
    ref = oracle.forward(**inp, mask_override=r_gpu, **okw)
    e_gpu = out["e"].cpu().numpy()
    de = np.abs(e_gpu - ref["e"]).max()
    assert de < E_TOL, de
    ref_r = (ref["e"] > tau.reshape(1, 1, H)).astype(bool)         # the oracle's own decisions
    near = np.abs(ref["e"] - tau.reshape(1, 1, H).astype(np.float64)) < NEAR
    assert not ((r_gpu.astype(bool) != ref_r) & ~near).any()
    assert rel_err_slices(np_of(out["S"]), ref["S"], 1) < 1e-4
    worst = {}
    for name in ("o", "o_rnn", "o_kv"):
        worst[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert worst[name] < TOL[torch.bfloat16], (name, worst[name])
    print(f"paper heads, every output: max|de|={de:.2e} worst slice errors {worst}")


def test_decode_fullsize_sampled_heads():
    """Decode at the full workload (batch 32, H=16, d=128, 32K-token prefix): 16 decode
    steps, then 64 sampled (sequence, head) pairs -- four of every head index, spread over
    the batch -- against one oracle pass over their whole prefix and steps (the pairs
    stacked along the oracle's batch axis, so its threads take one each)."""
    B, H, d, T0, steps = DECODE_B, DECODE_H, DECODE_D, DECODE_PREFIX, 16
    scale = d ** -0.5
    tau = np.full(H, 1.0, np.float32)        # a fixed threshold near the median score
    pre = make_inputs_torch(B, T0, H, d, dtype="bf16", seed=4, device=DEV)
    x = make_inputs_torch(steps, B, H, d, dtype="bf16", seed=5, device=DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    plan = ham.ForwardPlan(B, T0, H, d, d, torch.bfloat16, DEV, cap=T0 + steps, scale=scale)
    plan(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d)
    dplan = ham.DecodePlan(B, H, d, d, T0 + steps, torch.bfloat16, DEV, scale=scale)
    outs, es, rs = [], [], []
    for s in range(steps):
        dplan(x["q"][s], x["k"][s], x["v"][s], x["beta"][s], x["g"][s], tau_d, plan.S, plan.Kc,
              plan.Vc, plan.pos, plan.count, torch.full((B,), T0 + s, dtype=torch.int32, device=DEV))
        outs.append(np_of(dplan.o)); es.append(dplan.e.cpu().numpy()); rs.append(dplan.routed.cpu().numpy())
    torch.cuda.synchronize()
    assert int(dplan.status.item()) == 0
    e_pre = plan.e.cpu().numpy()
    r_pre = plan.routed.cpu().numpy()
    pairs = [((7 * h + 3 + 8 * j) % B, h) for h in range(H) for j in range(4)]
    n, T = len(pairs), T0 + steps
    sub = {nm: np.concatenate([np.concatenate([np_of(pre[nm][b:b + 1, :, h:h + 1]),
                                               np_of(x[nm][:, b, h]).reshape((1, steps, 1) + x[nm].shape[3:])],
                                              axis=1) for (b, h) in pairs], axis=0)
           for nm in ("q", "k", "v", "beta", "g")}
    emit = np.zeros((n, T, 1), np.int8)
    emit[:, T0:, 0] = 1
    e_all = np.stack([np.concatenate([e_pre[b, :, h], np.array([e[b, h] for e in es])]) for (b, h) in pairs])
    r_all = np.stack([np.concatenate([r_pre[b, :, h], np.array([r[b, h] for r in rs])])
                      for (b, h) in pairs]).astype(np.int8)
    ref = oracle.forward(**sub, tau=tau[:1], scale=scale, emit=emit)
    assert np.abs(e_all - ref["e"][:, :, 0]).max() < E_TOL
    near = np.abs(ref["e"][:, :, 0] - tau[0]) < NEAR
    assert not ((r_all.astype(bool) != ref["routed"][:, :, 0].astype(bool)) & ~near).any()
    if not np.array_equal(r_all, ref["routed"][:, :, 0]):
        ref = oracle.forward(**sub, tau=tau[:1], scale=scale, emit=emit, mask_override=r_all.reshape(n, T, 1))
    for i, (b, h) in enumerate(pairs):
        assert int(plan.count[b, h].item()) == int(ref["count"][i, 0])
        o_dec = np.stack([o[b, h] for o in outs])
        y = ref["o"][i, T0:, 0]
        err = np.abs(o_dec - y).max() / np.abs(y).max()
        assert err < TOL[torch.bfloat16], (b, h, err)
        errS = np.abs(np_of(plan.S[b, h]) - ref["S"][i, 0]).max() / np.abs(ref["S"][i, 0]).max()
        assert errS < 1e-4, (b, h, errS)


def test_decode_maximum_capacity_many_segments():
    """The largest cache the boundary accepts (cap = 4 194 304 entries per head, 2 GiB
    per K and V array here) with a ragged 70 001-token prefix, head 0 routing every
    token (70 001 cached keys: 69 split-K segments, more than one combine pass over
    the 64 lanes) and head 1 at a finite threshold; then decode steps against the
    oracle (attention outputs only at the decode steps)."""
    B, H, d, T0, steps = 1, 2, 128, 70001, 3
    cap = 4194304
    T = T0 + steps
    scale = d ** -0.5
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=45)
    tau = np.array([-np.inf, 1.0], np.float32)
    t = to_dev(inp, torch.bfloat16, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    plan = ham.ForwardPlan(B, T0, H, d, d, torch.bfloat16, DEV, cap=cap, scale=scale)
    plan(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau_d)
    dplan = ham.DecodePlan(B, H, d, d, cap, torch.bfloat16, DEV, scale=scale)
    outs, rs, es = [], [], []
    for s in range(steps):
        x = {n: t[n][:, T0 + s].contiguous() for n in t}
        dplan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau_d, plan.S, plan.Kc, plan.Vc, plan.pos,
              plan.count, torch.full((B,), T0 + s, dtype=torch.int32, device=DEV))
        outs.append(np_of(dplan.o)); rs.append(dplan.routed.cpu().numpy()); es.append(dplan.e.cpu().numpy())
    torch.cuda.synchronize()
    assert int(dplan.status.item()) == 0
    r_all = np.concatenate([plan.routed.cpu().numpy(), np.stack(rs, 1)], 1)
    e_all = np.concatenate([plan.e.cpu().numpy(), np.stack(es, 1)], 1)
    assert r_all[:, :, 0].all()
    emit = np.zeros((B, T, H), np.int8)
    emit[:, T0:] = 1
    ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, emit=emit)    # cap >= every count
    assert np.abs(e_all - ref["e"]).max() < E_TOL
    near = np.abs(ref["e"] - tau.reshape(1, 1, H).astype(np.float64)) < NEAR
    assert not ((r_all.astype(bool) != ref["routed"].astype(bool)) & ~near).any()
    if not np.array_equal(r_all.astype(bool), ref["routed"].astype(bool)):
        ref = oracle.forward(**inp, tau=tau, scale=scale, cap=T, emit=emit, mask_override=r_all)
    cnt = plan.count.cpu().numpy()
    assert np.array_equal(cnt, ref["count"]) and int(cnt[0, 0]) == T
    got = np.stack(outs, 1)
    assert rel_err_slices(got, ref["o"][:, T0:], 2) < TOL[torch.bfloat16]
    assert rel_err_slices(np_of(plan.S), ref["S"], 1) < 1e-4


@pytest.mark.parametrize("H,dk,dv,r,dkk", [(16, 128, 128, 2, 128), (5, 256, 384, 2, 128)])
def test_kv_heads_fullsize_sampled_heads(H, dk, dv, r, dkk):
    """The benchmark's head layouts at full size (B 8, T 4096, bf16): 32 KV heads of
    128/64 over the layer's 16 RNN heads, and the 800M layer's 5 RNN heads of 256/384
    with 10 KV heads of 128/192.  For sampled (sequence, RNN head) pairs the oracle runs
    that RNN head and its r KV heads over all tokens: every score, decision, cache entry
    of both KV heads and the final state, and the outputs at sampled tokens."""
    B, T = 8, 4096
    Hk, dvk = r * H, dv // r
    inp = make_inputs(B, T, H, dk, dv, dtype="bf16", seed=60 + dk)
    att = make_inputs(B, T, Hk, dkk, dvk, dtype="bf16", seed=61 + dk)
    tau = np.full(H, 1.0, np.float32)                  # routes about half of the tokens
    scale = dkk ** -0.5
    t, ta = to_dev(inp, torch.bfloat16, DEV), to_dev(att, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, q_attn=ta["q"], k_attn=ta["k"], v_attn=ta["v"], want_o_rnn=True,
                          want_o_kv=True)
    torch.cuda.synchronize()
    e_gpu = out["e"].cpu().numpy()
    r_gpu = out["routed"].cpu().numpy()
    cnt, pos = out["count"].cpu().numpy(), out["pos"].cpu().numpy()
    S = np_of(out["S"])
    rng = np.random.default_rng(62)
    for (b, h) in [(0, 0), (5, H - 1)]:
        sub = {n: np.ascontiguousarray(a[b:b + 1, :, h:h + 1]) for n, a in inp.items()}
        sa = {n: np.ascontiguousarray(a[b:b + 1, :, r * h:r * h + r]) for n, a in att.items()}
        toks = np.unique(np.concatenate([rng.choice(T, 24, replace=False), [0, T - 1]]))
        emit = np.zeros((1, T, 1), np.int8)
        emit[0, toks, 0] = 1
        okw = dict(tau=tau[h:h + 1], scale=scale, emit=emit, q_attn=sa["q"], k_attn=sa["k"], v_attn=sa["v"])
        ref = oracle.forward(**sub, **okw)
        de = np.abs(e_gpu[b, :, h] - ref["e"][0, :, 0]).max()
        assert de < E_TOL, (b, h, de)
        near = np.abs(ref["e"][0, :, 0] - tau[h]) < NEAR
        flips = r_gpu[b, :, h].astype(bool) != ref["routed"][0, :, 0].astype(bool)
        assert not (flips & ~near).any()
        if flips.any():
            ref = oracle.forward(**sub, mask_override=r_gpu[b:b + 1, :, h:h + 1], **okw)
        for i in range(r):
            j = r * h + i
            n = int(ref["count"][0, i])
            assert cnt[b, j] == n and np.array_equal(pos[b, j, :n], ref["pos"][0, i, :n])
        errS = np.abs(S[b, h] - ref["S"][0, 0]).max() / np.abs(ref["S"][0, 0]).max()
        assert errS < 1e-4, errS
        for name, heads in (("o", slice(h, h + 1)), ("o_rnn", slice(h, h + 1)), ("o_kv", slice(r * h, r * h + r))):
            x = np_of(out[name][b, toks, heads])
            y = ref[name][0, toks]
            err = np.abs(x - y).max() / max(np.abs(y).max(), 1e-30)
            assert err < TOL[torch.bfloat16], (name, b, h, err)
        print(f"kv heads H={H} dk={dk} dv={dv} (b={b}, h={h}): max|de|={de:.2e} flips={int(flips.sum())}")

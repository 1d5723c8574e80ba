"""Comparison protocol between the HIP library and the CPU oracle.

- Routing: the decision is bit-exact except for tokens whose oracle score lies
  within NEAR of tau (there the fp32 GPU score and the fp64 oracle score may fall
  on either side).  With block-contiguous routing the same holds per block, on
  the block's mean score.  Such tokens are counted and reported; the oracle is then re-run
  with the GPU's mask so that every output is compared on the same routed set.
- Compaction (count, pos, Kc, Vc): bit-exact.  With RoPE the cached keys are the
  rotated ones, computed in fp32 on the GPU and in fp64 by the oracle: Kc is then
  compared per slice at KC_ROPE_TOL (fp32 arithmetic; for bf16 one rounding of
  the rotated value, 2^-8 relative), pos and Vc still exactly.
- Floating outputs: per (b,h) slice, max|x - y| / max(max|y|, 1e-30) <= tol, with
  tol = 1e-4 for fp32 I/O and 2e-2 for bf16 I/O.  The fp32 state S_T is checked at
  1e-4 in both cases.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle

NEAR = 1e-5
E_TOL = 1e-5
TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
KC_ROPE_TOL = {torch.float32: 1e-5, torch.bfloat16: 8e-3}


def to_dev(inp, dtype, dev):
    out = {}
    for n, a in inp.items():
        t = torch.from_numpy(np.ascontiguousarray(a))
        if n in ("q", "k", "v", "q_attn", "k_attn", "v_attn"):
            t = t.to(dtype)
        out[n] = t.to(dev)
    return out


def np_of(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err_slices(x, y, head_axes):
    """max over (b,h) of max|x-y|/max|y| computed per head slice."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    worst = 0.0
    B = x.shape[0]
    H = x.shape[head_axes]
    for b in range(B):
        for h in range(H):
            xs = np.take(x[b], h, axis=head_axes - 1)
            ys = np.take(y[b], h, axis=head_axes - 1)
            den = max(np.abs(ys).max(), 1e-30)
            worst = max(worst, float(np.abs(xs - ys).max() / den))
    return worst


def block_means(e, n):
    """Mean of e [B,T,H] over aligned blocks of n tokens (complete blocks only),
    broadcast back to every token of the block; NaN for a trailing open block."""
    B, T, H = e.shape
    nb = T // n
    out = np.full((B, T, H), np.nan)
    out[:, :nb * n] = np.repeat(e[:, :nb * n].reshape(B, nb, n, H).mean(axis=2), n, axis=1)
    return out


def spread_block_flags(r, n):
    """Decode-step routing flags (1 at the last token of a routed block) to the
    forward's per-token form (every token of a routed block); an open trailing
    block is 0."""
    B, T, H = r.shape
    nb = T // n
    out = np.zeros_like(r)
    out[:, :nb * n] = np.repeat(r[:, n - 1:nb * n:n], n, axis=1)
    return out


def check_routing(e_gpu, r_gpu, ref, tau, route_block=0):
    """Returns (n_near_flips).  Asserts no flip outside the near band and |de| small.
    route_block > 1: blocks route on their mean score; tau at the block's last token."""
    H = e_gpu.shape[-1]
    e_ref = ref["e"]
    nan_ref = np.isnan(e_ref)                  # only learned-router scores can be NaN
    assert np.array_equal(np.isnan(e_gpu), nan_ref), "NaN scores differ"
    de = np.abs(e_gpu - e_ref)[~nan_ref]
    assert de.size == 0 or de.max() < E_TOL, f"score error {de.max():.3e}"
    t = np.asarray(tau, np.float64)
    t = t.reshape(1, 1, H) if t.size == H else t.reshape(e_ref.shape)   # per head or per token
    if route_block > 1:
        n = route_block
        t = np.broadcast_to(t, e_ref.shape)
        tl = np.zeros(e_ref.shape)
        nb = e_ref.shape[1] // n
        tl[:, :nb * n] = np.repeat(t[:, n - 1:nb * n:n], n, axis=1)
        near = np.abs(block_means(e_ref, n) - tl) < NEAR            # NaN (open block): False
    else:
        near = np.abs(e_ref - t) < NEAR
    flips = (r_gpu.astype(bool) != ref["routed"].astype(bool))
    bad = flips & ~near
    assert not bad.any(), f"{int(bad.sum())} routing flips outside the near band"
    return int((flips & near).sum())


def check_forward(out, inp, tau, dtype, *, scale, ref=None, gates=None, attn=None, S0=None,
                  cache=None, t0=0, eps=1e-6, check_outputs=("o", "o_rnn", "o_kv"), cap=None,
                  router_score=None, rope_base=0.0, doc_start=None, route_block=0):
    """Full comparison of one ham_forward result against the oracle.  With learned-router
    scores both sides compare the same float32 score with the same threshold, so the
    routing must match exactly (no near-threshold exemption)."""
    okw = dict(scale=scale, eps=eps, S0=S0, cache=cache, t0=t0, cap=cap, router_score=router_score,
               rope_base=rope_base, doc_start=doc_start, route_block=route_block)
    if gates is not None:
        okw.update(gate_rnn=gates[0], gate_kv=gates[1])
    if attn is not None:
        okw.update(q_attn=attn["q"], k_attn=attn["k"], v_attn=attn["v"])
    if ref is None:
        ref = oracle.forward(**inp, tau=tau, **okw)
    e_gpu = out["e"].cpu().numpy()
    r_gpu = out["routed"].cpu().numpy()
    nflip = check_routing(e_gpu, r_gpu, ref, tau, route_block)
    if router_score is not None and route_block <= 1:
        assert np.array_equal(e_gpu, np.asarray(router_score, np.float32), equal_nan=True)
        assert nflip == 0 and np.array_equal(r_gpu.astype(bool), ref["routed"].astype(bool))
    if nflip:
        ref = oracle.forward(**inp, tau=tau, mask_override=r_gpu, **okw)
    tol = TOL[dtype]
    cnt = out["count"].cpu().numpy()
    assert np.array_equal(cnt, ref["count"]), (cnt, ref["count"])
    pos = out["pos"].cpu().numpy()
    Kc, Vc = np_of(out["Kc"]), np_of(out["Vc"])
    B, H = cnt.shape
    for b in range(B):
        for h in range(H):
            n = cnt[b, h]
            assert np.array_equal(pos[b, h, :n], ref["pos"][b, h, :n])
            if rope_base > 0:
                if n:
                    kr = ref["Kc"][b, h, :n]
                    dk = np.abs(Kc[b, h, :n] - kr).max() / max(np.abs(kr).max(), 1e-30)
                    assert dk < KC_ROPE_TOL[dtype], (b, h, dk)
            else:
                assert np.array_equal(Kc[b, h, :n], ref["Kc"][b, h, :n])
            assert np.array_equal(Vc[b, h, :n], ref["Vc"][b, h, :n])
    errs = {"S": rel_err_slices(np_of(out["S"]), ref["S"], 1)}
    assert errs["S"] < 1e-4, errs
    for name in check_outputs:
        if out.get(name) is None:
            continue
        errs[name] = rel_err_slices(np_of(out[name]), ref[name], 2)
        assert errs[name] < tol, (name, errs)
    return dict(ref=ref, nflip=nflip, errs=errs)

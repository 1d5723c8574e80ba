"""HAM (Hybrid Associative Memory) sequence mixer on AMD MI355X.

Python binding of the C ABI in include/ham.h.  This module only marshals
arguments: it checks shapes and dtypes of torch tensors, allocates outputs and
scratch with torch (device memory plumbing), and passes raw device pointers and
the current HIP stream to libham.so.  Every step of the layer runs in the HIP
kernels of that library; if it is missing, the calls raise.

Method: "Hybrid Associative Memories" (arXiv 2603.22325), §2 and App. A.1.
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import (HAM_BF16, HAM_CONTINUE, HAM_EXTERNAL_SCORES, HAM_F32, HAM_FORCE_RECURRENT,
                   HAM_OVERLAP, HAM_TAU_PER_TOKEN, HamDims, HamError, check)

__all__ = ["ham_forward", "ham_decode_step", "ham_route_stats", "ham_select_tau", "ForwardPlan",
           "DecodePlan", "HamError", "HAM_CONTINUE", "HAM_FORCE_RECURRENT", "HAM_EXTERNAL_SCORES",
           "HAM_TAU_PER_TOKEN", "HAM_OVERLAP", "library_path"]

library_path = _lib.LIB_PATH


def _vp(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _io_code(dtype):
    if dtype == torch.float32:
        return HAM_F32
    if dtype == torch.bfloat16:
        return HAM_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(name, t, shape, dtype, device):
    if t is None:
        return None
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype} != expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _tau_flag(tau, per_token_shape, dev):
    """0 for a per-head threshold [H], HAM_TAU_PER_TOKEN for one per token and head."""
    if tau is None:
        raise ValueError("tau is required")
    H = per_token_shape[-1]
    if tuple(tau.shape) == tuple(per_token_shape):
        _need("tau", tau, per_token_shape, torch.float32, dev)
        return HAM_TAU_PER_TOKEN
    _need("tau", tau, (H,), torch.float32, dev)
    return 0


def make_dims(B, T, H, dk, dv, io, scale, eps, cap, flags=0, t0=0, rope_base=0.0, route_block=0,
              kv=None):
    """kv: None, or (kv_heads, dk_kv, dv_kv) of attention heads with their own geometry."""
    kh, kdk, kdv = kv if kv is not None else (0, 0, 0)
    return HamDims(B, T, H, dk, dv, io, float(scale), float(eps), cap, flags, t0, float(rope_base),
                   int(route_block), int(kh), int(kdk), int(kdv))


def _kv_geometry(H, dk, dv, kv):
    """(kv_heads, dk_kv, dv_kv), defaulting to the RNN heads' geometry."""
    if kv is None:
        return H, dk, dv
    kh, kdk, kdv = kv
    return kh or H, kdk or dk, kdv or dv


class ForwardPlan:
    """Outputs and scratch for repeated ham_forward calls of one shape.

    Allocation happens once here; each call only enqueues the kernels.
    """

    def __init__(self, B, T, H, dk, dv, dtype, device, *, cap=None, scale=None,
                 norm_eps=1e-6, flags=0, t0=0, rope_base=0.0, route_block=0, kv_heads=0, dk_kv=0,
                 dv_kv=0, want_o_rnn=False, want_o_kv=False):
        """kv_heads, dk_kv, dv_kv: attention (KV) heads with their own geometry (0: the
        RNN heads'); the cache, gate_kv, o_kv and q_attn/k_attn/v_attn are then shaped
        [.., kv_heads, dk_kv|dv_kv]."""
        device = torch.device(device)
        self.io = _io_code(dtype)
        self.dtype, self.device = dtype, device
        self.cap = T if cap is None else cap
        self.scale = 1.0 / math.sqrt(dk) if scale is None else scale
        kv = (kv_heads, dk_kv, dv_kv)
        self.dims = make_dims(B, T, H, dk, dv, self.io, self.scale, norm_eps, self.cap, flags, t0,
                              rope_base, route_block, kv)
        self.shape = (B, T, H, dk, dv)
        self.kv = _kv_geometry(H, dk, dv, kv)
        HK, DKK, DVK = self.kv
        L = _lib.lib()
        ws_bytes = L.ham_forward_workspace_size(ctypes.byref(self.dims))
        if ws_bytes == 0:
            raise HamError(-1, L.ham_last_error().decode())
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.o = torch.empty((B, T, H, dv), dtype=dtype, device=device)
        self.o_rnn = torch.empty((B, T, H, dv), dtype=dtype, device=device) if want_o_rnn else None
        self.o_kv = torch.empty((B, T, HK, DVK), dtype=dtype, device=device) if want_o_kv else None
        self.e = torch.empty((B, T, H), dtype=torch.float32, device=device)
        self.routed = torch.empty((B, T, H), dtype=torch.uint8, device=device)
        self.S = torch.empty((B, H, dk, dv), dtype=torch.float32, device=device)
        self.Kc = torch.zeros((B, HK, self.cap, DKK), dtype=dtype, device=device)
        self.Vc = torch.zeros((B, HK, self.cap, DVK), dtype=dtype, device=device)
        self.pos = torch.full((B, HK, self.cap), -1, dtype=torch.int32, device=device)
        self.count = torch.zeros((B, HK), dtype=torch.int32, device=device)

    def __call__(self, q, k, v, beta, g, tau, *, q_attn=None, k_attn=None, v_attn=None,
                 gate_rnn=None, gate_kv=None, S0=None, router_scores=None, doc_start=None,
                 stream=None):
        """router_scores: [B,T,H] float32 scores of a learned router, which then replace
        the RNN's prediction error as the routing score (needs the plan to have been
        made with flags including HAM_EXTERNAL_SCORES).  doc_start: [B,T] int32
        absolute start position of each token's document in a packed batch (the
        attention then sees only keys of the same document), or None."""
        B, T, H, dk, dv = self.shape
        HK, DKK, DVK = self.kv
        dev, dt = self.device, self.dtype
        for n, t in (("q", q), ("k", k)):
            _need(n, t, (B, T, H, dk), dt, dev)
        _need("v", v, (B, T, H, dv), dt, dev)
        for n, t in (("q_attn", q_attn), ("k_attn", k_attn)):
            _need(n, t, (B, T, HK, DKK), dt, dev)
        _need("v_attn", v_attn, (B, T, HK, DVK), dt, dev)
        for n, t in (("beta", beta), ("g", g), ("gate_rnn", gate_rnn)):
            _need(n, t, (B, T, H), torch.float32, dev)
        _need("gate_kv", gate_kv, (B, T, HK), torch.float32, dev)
        tf = _tau_flag(tau, (B, T, H), dev)
        self.dims.flags = (self.dims.flags & ~HAM_TAU_PER_TOKEN) | tf
        _need("S0", S0, (B, H, dk, dv), torch.float32, dev)
        _need("doc_start", doc_start, (B, T), torch.int32, dev)
        if q is None or k is None or v is None or beta is None or g is None or tau is None:
            raise ValueError("q, k, v, beta, g and tau are required")
        ext = bool(self.dims.flags & HAM_EXTERNAL_SCORES)
        if ext != (router_scores is not None):
            raise ValueError("router_scores must be given exactly when the plan has HAM_EXTERNAL_SCORES")
        if ext:
            self.e = _need("router_scores", router_scores, (B, T, H), torch.float32, dev)
        rc = _lib.lib().ham_forward(
            ctypes.byref(self.dims), _vp(q), _vp(k), _vp(v), _vp(q_attn), _vp(k_attn), _vp(v_attn),
            _vp(beta), _vp(g), _vp(tau), _vp(gate_rnn), _vp(gate_kv), _vp(doc_start), _vp(S0), _vp(self.S),
            _vp(self.o), _vp(self.o_rnn), _vp(self.o_kv), _vp(self.e), _vp(self.routed),
            _vp(self.Kc), _vp(self.Vc), _vp(self.pos), _vp(self.count),
            _vp(self.ws), self.ws.numel(), _stream(stream))
        check(rc)
        return self

    def result(self):
        return dict(o=self.o, o_rnn=self.o_rnn, o_kv=self.o_kv, e=self.e, routed=self.routed,
                    S=self.S, Kc=self.Kc, Vc=self.Vc, pos=self.pos, count=self.count)


def ham_forward(q, k, v, beta, g, tau, *, scale=None, norm_eps=1e-6, cap=None, q_attn=None,
                k_attn=None, v_attn=None, gate_rnn=None, gate_kv=None, S0=None, cache=None,
                t0=0, force_recurrent=False, router_scores=None, rope_base=0.0, doc_start=None,
                route_block=0, want_o_rnn=False, want_o_kv=False, overlap=False, stream=None):
    """One HAM layer over q, k, v [B,T,H,d] (float32 or bfloat16, on the GPU).

    tau: [H] float32 thresholds per head, or [B,T,H] per token and head (a schedule
    along the sequence that steers how the cache grows).

    cache: None, or dict(Kc, Vc, pos, count) of an earlier call to continue; it
    is then extended in place and S0 should be that call's state.  router_scores:
    None, or [B,T,H] float32 scores of a learned router that replace the RNN's
    prediction error as the routing score (tau then in the router's units).
    rope_base: 0, or the RoPE base for the attention-path query and key (the cache
    then holds rotated keys).  doc_start: None, or [B,T] int32 absolute start
    positions of the tokens' documents (same-document masking of a packed batch).
    route_block: 0 (per-token routing), or 2..64 (a power of two) for block-contiguous
    routing: aligned blocks route whole on their mean score and become visible from
    their last token on; t0 and T must then be multiples of it.  overlap: with
    router_scores, run the RNN on the library's second stream beside the routing and
    attention (HAM_OVERLAP).  Returns a dict with
    o, e, routed, S, Kc, Vc, pos, count (and o_rnn / o_kv if asked); e is the routing
    score used.
    """
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flags = ((HAM_FORCE_RECURRENT if force_recurrent else 0) | (HAM_CONTINUE if cache is not None else 0)
             | (HAM_EXTERNAL_SCORES if router_scores is not None else 0) | (HAM_OVERLAP if overlap else 0))
    if cache is not None:
        cap = cache["Kc"].shape[2]
    # the attention heads take the geometry of the attention-path inputs
    HK, DKK, DVK = (q_attn.shape[2], q_attn.shape[3], v_attn.shape[3]) if (
        q_attn is not None and v_attn is not None) else (H, dk, dv)
    plan = ForwardPlan(B, T, H, dk, dv, q.dtype, q.device, cap=cap, scale=scale,
                       norm_eps=norm_eps, flags=flags, t0=t0, rope_base=rope_base,
                       route_block=route_block, kv_heads=HK, dk_kv=DKK, dv_kv=DVK,
                       want_o_rnn=want_o_rnn, want_o_kv=want_o_kv)
    if cache is not None:
        plan.Kc = _need("Kc", cache["Kc"], (B, HK, plan.cap, DKK), q.dtype, q.device)
        plan.Vc = _need("Vc", cache["Vc"], (B, HK, plan.cap, DVK), q.dtype, q.device)
        plan.pos = _need("pos", cache["pos"], (B, HK, plan.cap), torch.int32, q.device)
        plan.count = _need("count", cache["count"], (B, HK), torch.int32, q.device)
    plan(q, k, v, beta, g, tau, q_attn=q_attn, k_attn=k_attn, v_attn=v_attn,
         gate_rnn=gate_rnn, gate_kv=gate_kv, S0=S0, router_scores=router_scores,
         doc_start=doc_start, stream=stream)
    return plan.result()


class DecodePlan:
    """Scratch and outputs for repeated ham_decode_step calls on one cache."""

    def __init__(self, B, H, dk, dv, cap, dtype, device, *, scale=None, norm_eps=1e-6,
                 rope_base=0.0, route_block=0, kv_heads=0, dk_kv=0, dv_kv=0, want_o_rnn=False,
                 want_o_kv=False, noalloc=False):
        """noalloc: call ham_decode_step_noalloc, whose scratch is the library's fixed
        per-GPU array (no workspace is allocated here; steps that need more than it
        holds are rejected)."""
        device = torch.device(device)
        self.noalloc = noalloc
        self.io = _io_code(dtype)
        self.dtype, self.device = dtype, device
        self.scale = 1.0 / math.sqrt(dk) if scale is None else scale
        kv = (kv_heads, dk_kv, dv_kv)
        self.dims = make_dims(B, 1, H, dk, dv, self.io, self.scale, norm_eps, cap, rope_base=rope_base,
                              route_block=route_block, kv=kv)
        self.kv = _kv_geometry(H, dk, dv, kv)
        # block-contiguous routing: the open block's running score sum per (b, h)
        self.block_score = (torch.zeros((B, H), dtype=torch.float32, device=device)
                            if route_block > 1 else None)
        self.shape = (B, H, dk, dv, cap)
        L = _lib.lib()
        ws_bytes = L.ham_decode_workspace_size(ctypes.byref(self.dims))
        if ws_bytes == 0:
            raise HamError(-1, L.ham_last_error().decode())
        self.ws = None if noalloc else torch.empty(ws_bytes, dtype=torch.uint8, device=device)
        self.o = torch.empty((B, H, dv), dtype=dtype, device=device)
        self.o_rnn = torch.empty((B, H, dv), dtype=dtype, device=device) if want_o_rnn else None
        self.o_kv = (torch.empty((B, self.kv[0], self.kv[2]), dtype=dtype, device=device)
                     if want_o_kv else None)
        self.e = torch.empty((B, H), dtype=torch.float32, device=device)
        self.routed = torch.empty((B, H), dtype=torch.uint8, device=device)
        self.status = torch.zeros((1,), dtype=torch.int32, device=device)

    def __call__(self, q, k, v, beta, g, tau, S, Kc, Vc, pos, count, t_abs, *, q_attn=None,
                 k_attn=None, v_attn=None, gate_rnn=None, gate_kv=None, router_scores=None,
                 doc_start=None, block_score=None, stream=None):
        """router_scores: None, or [B,H] float32 learned-router scores of the new tokens,
        which then replace the RNN's prediction error as the routing score.
        doc_start: None, or [B] int32 absolute start of each new token's document.
        block_score: with block-contiguous routing, the [B,H] float32 running score sum
        of the open blocks (default: the plan's own, zero at creation)."""
        B, H, dk, dv, cap = self.shape
        HK, DKK, DVK = self.kv
        dev, dt = self.device, self.dtype
        for n, t in (("q", q), ("k", k)):
            _need(n, t, (B, H, dk), dt, dev)
        _need("v", v, (B, H, dv), dt, dev)
        for n, t in (("q_attn", q_attn), ("k_attn", k_attn)):
            _need(n, t, (B, HK, DKK), dt, dev)
        _need("v_attn", v_attn, (B, HK, DVK), dt, dev)
        for n, t in (("beta", beta), ("g", g), ("gate_rnn", gate_rnn)):
            _need(n, t, (B, H), torch.float32, dev)
        _need("gate_kv", gate_kv, (B, HK), torch.float32, dev)
        tf = _tau_flag(tau, (B, H), dev)
        _need("S", S, (B, H, dk, dv), torch.float32, dev)
        _need("Kc", Kc, (B, HK, cap, DKK), dt, dev)
        _need("Vc", Vc, (B, HK, cap, DVK), dt, dev)
        _need("pos", pos, (B, HK, cap), torch.int32, dev)
        _need("count", count, (B, HK), torch.int32, dev)
        _need("t_abs", t_abs, (B,), torch.int32, dev)
        _need("router_scores", router_scores, (B, H), torch.float32, dev)
        _need("doc_start", doc_start, (B,), torch.int32, dev)
        if block_score is None:
            block_score = self.block_score
        _need("block_score", block_score, (B, H), torch.float32, dev)
        self.dims.flags = (HAM_EXTERNAL_SCORES if router_scores is not None else 0) | tf
        e = router_scores if router_scores is not None else self.e
        args = [ctypes.byref(self.dims), _vp(q), _vp(k), _vp(v), _vp(q_attn), _vp(k_attn), _vp(v_attn),
                _vp(beta), _vp(g), _vp(tau), _vp(gate_rnn), _vp(gate_kv), _vp(doc_start),
                _vp(block_score), _vp(S), _vp(Kc), _vp(Vc),
                _vp(pos), _vp(count), _vp(t_abs), _vp(self.o), _vp(self.o_rnn), _vp(self.o_kv),
                _vp(e), _vp(self.routed), _vp(self.status)]
        if self.noalloc:
            rc = _lib.lib().ham_decode_step_noalloc(*args, _stream(stream))
        else:
            rc = _lib.lib().ham_decode_step(*args, _vp(self.ws), self.ws.numel(), _stream(stream))
        check(rc)
        return self


def ham_decode_step(q, k, v, beta, g, tau, S, cache, t_abs, *, scale=None, norm_eps=1e-6,
                    q_attn=None, k_attn=None, v_attn=None, gate_rnn=None, gate_kv=None,
                    rope_base=0.0, doc_start=None, route_block=0, want_o_rnn=False, want_o_kv=False,
                    stream=None):
    """One decode step: q, k, v [B,H,d]; tau [H] or [B,H]; S and cache (dict Kc, Vc, pos, count) are
    updated in place; t_abs [B] int32 positions (also the RoPE positions when
    rope_base > 0).  With route_block > 1 the cache dict also carries the open
    blocks' score sums as cache["block_score"] ([B,H] float32, added as zeros if
    missing).  Returns dict(o, e, routed, status, ...)."""
    B, H, dk = q.shape
    dv = v.shape[-1]
    cap = cache["Kc"].shape[2]
    HK, DKK, DVK = (q_attn.shape[1], q_attn.shape[2], v_attn.shape[2]) if (
        q_attn is not None and v_attn is not None) else (H, dk, dv)
    plan = DecodePlan(B, H, dk, dv, cap, q.dtype, q.device, scale=scale, norm_eps=norm_eps,
                      rope_base=rope_base, route_block=route_block, kv_heads=HK, dk_kv=DKK,
                      dv_kv=DVK, want_o_rnn=want_o_rnn, want_o_kv=want_o_kv)
    if route_block > 1 and "block_score" not in cache:
        cache["block_score"] = plan.block_score
    plan(q, k, v, beta, g, tau, S, cache["Kc"], cache["Vc"], cache["pos"], cache["count"], t_abs,
         q_attn=q_attn, k_attn=k_attn, v_attn=v_attn, gate_rnn=gate_rnn, gate_kv=gate_kv,
         doc_start=doc_start, block_score=cache.get("block_score") if route_block > 1 else None,
         stream=stream)
    return dict(o=plan.o, o_rnn=plan.o_rnn, o_kv=plan.o_kv, e=plan.e, routed=plan.routed,
                status=plan.status)


def ham_route_stats(k, v, beta, g, tau, *, q=None, S0=None, near_band=1e-5, want_rho=True,
                    force_recurrent=False, route_block=0, stream=None):
    """Routing only (RNN scores, threshold, counts).  Returns dict(e, routed, count,
    n_near, rho); rho is None unless want_rho (which waits for the stream).  With
    route_block > 1 (block-contiguous routing) n_near is not computed (None)."""
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    dev, dt = k.device, k.dtype
    io = _io_code(dt)
    _need("v", v, (B, T, H, dv), dt, dev)
    _need("beta", beta, (B, T, H), torch.float32, dev)
    _need("g", g, (B, T, H), torch.float32, dev)
    tf = _tau_flag(tau, (B, T, H), dev)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev)
    dims = make_dims(B, T, H, dk, dv, io, 1.0, 1e-6, max(T, 1),
                     (HAM_FORCE_RECURRENT if force_recurrent else 0) | tf, route_block=route_block)
    L = _lib.lib()
    ws_bytes = L.ham_route_stats_workspace_size(ctypes.byref(dims))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    e = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    routed = torch.empty((B, T, H), dtype=torch.uint8, device=dev)
    count = torch.empty((B, H), dtype=torch.int32, device=dev)
    n_near = torch.empty((H,), dtype=torch.int64, device=dev) if route_block <= 1 else None
    rho = ctypes.c_double(float("nan"))
    rc = L.ham_route_stats(ctypes.byref(dims), _vp(q), _vp(k), _vp(v), _vp(beta), _vp(g), _vp(tau),
                           _vp(S0), _vp(e), _vp(routed), _vp(count), _vp(n_near),
                           ctypes.c_float(near_band), ctypes.byref(rho) if want_rho else None,
                           _vp(ws), ws.numel(), _stream(stream))
    check(rc)
    return dict(e=e, routed=routed, count=count, n_near=n_near, rho=rho.value if want_rho else None)


def ham_select_tau(e, rho, *, out=None, stream=None):
    """Per-head threshold [H] float32 that routes round(rho*B*T) of each head's scores
    e [B,T,H] (float32, on the GPU): the midpoint of the two order statistics around
    the cut; +inf for rho*N rounding to 0, -inf for N."""
    B, T, H = e.shape
    _need("e", e, (B, T, H), torch.float32, e.device)
    tau = torch.empty((H,), dtype=torch.float32, device=e.device) if out is None else out
    _need("out", tau, (H,), torch.float32, e.device)
    dims = make_dims(B, T, H, 64, 64, HAM_F32, 1.0, 1e-6, max(T, 1))
    rc = _lib.lib().ham_select_tau(ctypes.byref(dims), _vp(e), ctypes.c_double(float(rho)), _vp(tau),
                                   _stream(stream))
    check(rc)
    return tau


def ham_attention_backward(q_attn, cache, dO, *, scale=None, t0=0, doc_start=None, stream=None):
    """Gradients of the attention readout o_kv for training: q_attn [B,T,H,dk] (the
    forward's attention-path queries), cache dict(Kc, Vc, pos, count) as the forward
    left it, dO [B,T,H,dv] float32 = dL/do_kv.  Returns dict(dq [B,T,H,dk],
    dKc [B,H,cap,dk], dVc [B,H,cap,dv]) in float32 (cache rows < count)."""
    B, T, H, dk = q_attn.shape
    Kc, Vc, pos, count = cache["Kc"], cache["Vc"], cache["pos"], cache["count"]
    cap, dv = Kc.shape[2], Vc.shape[3]
    dev, dt = q_attn.device, q_attn.dtype
    _need("q_attn", q_attn, (B, T, H, dk), dt, dev)
    _need("Kc", Kc, (B, H, cap, dk), dt, dev)
    _need("Vc", Vc, (B, H, cap, dv), dt, dev)
    _need("pos", pos, (B, H, cap), torch.int32, dev)
    _need("count", count, (B, H), torch.int32, dev)
    _need("dO", dO, (B, T, H, dv), torch.float32, dev)
    _need("doc_start", doc_start, (B, T), torch.int32, dev)
    scale = 1.0 / math.sqrt(dk) if scale is None else scale
    dims = make_dims(B, T, H, dk, dv, _io_code(dt), scale, 1e-6, cap, t0=t0)
    L = _lib.lib()
    ws_bytes = L.ham_attention_backward_workspace_size(ctypes.byref(dims))
    if ws_bytes == 0:
        raise HamError(-1, L.ham_last_error().decode())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    dq = torch.empty((B, T, H, dk), dtype=torch.float32, device=dev)
    dKc = torch.zeros((B, H, cap, dk), dtype=torch.float32, device=dev)
    dVc = torch.zeros((B, H, cap, dv), dtype=torch.float32, device=dev)
    check(L.ham_attention_backward(ctypes.byref(dims), _vp(q_attn), _vp(Kc), _vp(Vc), _vp(pos), _vp(count),
                                   _vp(doc_start), _vp(dO), _vp(dq), _vp(dKc), _vp(dVc), _vp(ws), ws.numel(),
                                   _stream(stream)))
    return dict(dq=dq, dKc=dKc, dVc=dVc)


def ham_rnn_backward(q, k, v, beta, g, dO, *, S0=None, dS_T=None, force_recurrent=False, stream=None):
    """Gradients of the gated delta-rule RNN for training: q, k [B,T,H,dk], v [B,T,H,dv]
    (float32 or bfloat16), beta, g [B,T,H] float32 (the forward's inputs), S0 the
    forward's entering state or None, dO = dL/do_rnn [B,T,H,dv] float32, dS_T = dL/dS_T
    [B,H,dk,dv] or None.  The chunked form runs unless force_recurrent asks for the
    token-serial reverse (HAM_FORCE_RECURRENT).  Returns dict(dq, dk, dv, dbeta, dg, dS0)
    in float32."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    dev, dt = q.device, q.dtype
    _need("k", k, (B, T, H, dk), dt, dev)
    _need("v", v, (B, T, H, dv), dt, dev)
    for n, t in (("beta", beta), ("g", g)):
        _need(n, t, (B, T, H), torch.float32, dev)
    _need("dO", dO, (B, T, H, dv), torch.float32, dev)
    _need("S0", S0, (B, H, dk, dv), torch.float32, dev)
    _need("dS_T", dS_T, (B, H, dk, dv), torch.float32, dev)
    dims = make_dims(B, T, H, dk, dv, _io_code(dt), 1.0, 1e-6, max(T, 1),
                     flags=HAM_FORCE_RECURRENT if force_recurrent else 0)
    L = _lib.lib()
    ws_bytes = L.ham_rnn_backward_workspace_size(ctypes.byref(dims))
    if ws_bytes == 0:
        raise HamError(-2, L.ham_last_error().decode())
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = dict(dq=torch.empty((B, T, H, dk), dtype=torch.float32, device=dev),
               dk=torch.empty((B, T, H, dk), dtype=torch.float32, device=dev),
               dv=torch.empty((B, T, H, dv), dtype=torch.float32, device=dev),
               dbeta=torch.empty((B, T, H), dtype=torch.float32, device=dev),
               dg=torch.empty((B, T, H), dtype=torch.float32, device=dev),
               dS0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev))
    check(L.ham_rnn_backward(ctypes.byref(dims), _vp(q), _vp(k), _vp(v), _vp(beta), _vp(g), _vp(S0),
                             _vp(dO), _vp(dS_T), _vp(out["dq"]), _vp(out["dk"]), _vp(out["dv"]),
                             _vp(out["dbeta"]), _vp(out["dg"]), _vp(out["dS0"]), _vp(ws), ws.numel(),
                             _stream(stream)))
    return out

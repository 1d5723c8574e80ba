"""CPU oracle of one HAM layer (fp64, token-serial).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product path (the
HIP library and its Python binding) never imports, loads or calls anything here,
and nothing here imports the product package.

The arithmetic lives in ``ham_oracle.c`` (plain C, double precision); this module
only compiles it with gcc, converts arrays to float64 and splits independent
heads over threads.  Source of the method: "Hybrid Associative Memories"
(arXiv 2603.22325, full-text page) -- §2 for the KV memory, DeltaNet update,
routing score and gated mix; App. A.1 for the state orientation, the fit-error
router, masking by original position and generation.

Every function here is pinned by tests/test_oracle_pins.py against closed forms,
invariants, textbook linear algebra and brute force.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ham_oracle.c")
_LIB = os.path.join(_HERE, "libham_oracle.so")
_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile ham_oracle.c with gcc (no fast-math: IEEE double throughout)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if (not os.path.exists(_LIB)) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.ham_oracle_forward.restype = ctypes.c_int
        lib.ham_oracle_forward.argtypes = (
            [ctypes.c_int] * 8 + [ctypes.c_double] * 3 + [ctypes.c_int] + [P] * 3 + [P] * 3 + [P] * 3
            + [P] * 2 + [P] * 5 + [P, ctypes.c_int, P, P, P, P] + [P] * 5
            + [ctypes.c_int, ctypes.c_int])
        _lib = lib
        return lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def forward(q, k, v, beta, g, tau, *, scale, eps=1e-6, rope_base=0.0, q_attn=None, k_attn=None,
            v_attn=None, gate_rnn=None, gate_kv=None, mask_override=None, router_score=None,
            S0=None, cache=None, cap=None, t0=0, doc_start=None, emit=None, route_block=0,
            threads=None):
    """Run the oracle over all heads.

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta, g: [B,T,H]; tau: [H] per head, or [B,T,H]
    per token and head (a threshold schedule along the sequence); float32, e-units.
    S0: [B,H,dk,dv] or None (zeros).  cache: None or dict(Kc, Vc, pos, count) of an
    existing cache to continue ([B,H,cap,d], [B,H,cap], [B,H]).  t0: int or [B]
    absolute position of token 0.  rope_base: 0, or the RoPE base applied to the
    attention-path query and key at their positions (the cache holds rotated keys).
    doc_start: None or [B,T] int, the absolute position where each token's document
    begins in a packed batch (attention only to cached keys at positions >= it).
    router_score: None or [B,T,H] float32 scores of a
    learned router that replace the fit-error score (the decision is score > tau).
    emit: None or [B,T,H] bool; False skips the
    attention readout and mix of that token (o_kv, o stay 0).  route_block: 0 or 1
    (per-token routing), or n > 1 for block-contiguous routing ([HAM] §7): aligned
    blocks of n positions route whole on float(mean of their scores) > tau at the
    block's last token and enter the cache at that token (t0 must be a multiple of
    n; a block still open at the end stays unrouted).  Attention heads of their own
    geometry ([HAM] §4 model setup: twice the RNN heads, half their size): given by
    q_attn [B,T,Hk,dkk] and v_attn [B,T,Hk,dvk] with Hk = r*H and r*dvk = dv; KV head
    r*h + i follows RNN head h's routing; gate_kv is then [B,T,Hk], the cache and o_kv
    are per KV head.  Returns a dict of float64 / int arrays:
    e, routed, o_rnn, o_kv, o, S, Kc, Vc, pos, count.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    beta, g = _f64(beta), _f64(g)
    qa, ka, va = _f64(q_attn), _f64(k_attn), _f64(v_attn)
    gr, gk = _f64(gate_rnn), _f64(gate_kv)
    Hk, dkk, dvk = (qa.shape[2], qa.shape[3], va.shape[3]) if (qa is not None and va is not None) \
        else (H, dk, dv)
    tau = np.asarray(tau, dtype=np.float32)
    tau = np.ascontiguousarray(np.broadcast_to(tau.reshape(H) if tau.size == H else tau.reshape(B, T, H),
                                               (B, T, H)))
    mo = None if mask_override is None else np.ascontiguousarray(
        np.asarray(mask_override).astype(np.int8))
    rs = None if router_score is None else np.ascontiguousarray(
        np.asarray(router_score, dtype=np.float32).reshape(B, T, H))
    em = None if emit is None else np.ascontiguousarray(np.asarray(emit).astype(np.int8))
    t0a = np.ascontiguousarray(np.broadcast_to(np.asarray(t0, dtype=np.int64), (B,)))
    dc = None if doc_start is None else np.ascontiguousarray(
        np.asarray(doc_start, dtype=np.int64).reshape(B, T))
    S = np.zeros((B, H, dk, dv)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    S = np.ascontiguousarray(S)
    if cache is None:
        cap = T if cap is None else cap
        Kc = np.zeros((B, Hk, cap, dkk))
        Vc = np.zeros((B, Hk, cap, dvk))
        pos = np.full((B, Hk, cap), -1, dtype=np.int64)
        count = np.zeros((B, Hk), dtype=np.int64)
    else:
        Kc = np.array(cache["Kc"], dtype=np.float64, copy=True)
        Vc = np.array(cache["Vc"], dtype=np.float64, copy=True)
        pos = np.array(cache["pos"], dtype=np.int64, copy=True)
        count = np.array(cache["count"], dtype=np.int64, copy=True)
        cap = Kc.shape[2]
    Kc, Vc, pos, count = (np.ascontiguousarray(a) for a in (Kc, Vc, pos, count))
    e = np.zeros((B, T, H))
    routed = np.zeros((B, T, H), dtype=np.int8)
    o_rnn = np.zeros((B, T, H, dv))
    o_kv = np.zeros((B, T, Hk, dvk))
    o = np.zeros((B, T, H, dv))

    lib = _load()
    nheads = B * H
    nthr = max(1, min(threads or default_threads(), nheads))
    bounds = [nheads * i // nthr for i in range(nthr + 1)]

    def run(i):
        return lib.ham_oracle_forward(
            B, T, H, dk, dv, Hk, dkk, dvk, float(scale), float(eps), float(rope_base), int(route_block),
            _ptr(q), _ptr(k), _ptr(v), _ptr(qa), _ptr(ka), _ptr(va),
            _ptr(beta), _ptr(g), _ptr(tau), _ptr(gr), _ptr(gk), _ptr(mo), _ptr(rs), _ptr(em),
            _ptr(t0a), _ptr(dc),
            _ptr(S), cap, _ptr(Kc), _ptr(Vc), _ptr(pos), _ptr(count),
            _ptr(e), _ptr(routed), _ptr(o_rnn), _ptr(o_kv), _ptr(o),
            bounds[i], bounds[i + 1])

    if nthr == 1:
        rcs = [run(0)]
    else:
        with ThreadPoolExecutor(nthr) as ex:
            rcs = list(ex.map(run, range(nthr)))
    if any(rc == -1 for rc in rcs):
        raise ValueError("oracle: t0 must be a multiple of route_block, and the attention heads "
                         "must tile the RNN heads (Hk = r*H, r*dvk = dv, own q/k/v_attn)")
    if any(rc != 0 for rc in rcs):
        raise RuntimeError("oracle: KV cache capacity exceeded")
    return dict(e=e, routed=routed, o_rnn=o_rnn, o_kv=o_kv, o=o, S=S, Kc=Kc, Vc=Vc,
                pos=pos, count=count)


def select_tau(e, rho):
    """Per-head threshold for a target KV fraction rho ([HAM] §5: rho_KV, the share of
    a layer's tokens kept in the KV cache; App. A.1 "Forward Pass": a token is stored
    when its score exceeds the threshold).  For head h the N = B*T scores e[:, :, h]
    are sorted ascending (NaN last); k = round(rho * N) (Python's round: nearest,
    ties to even); tau = +inf for k = 0, -inf for k = N, otherwise the float32 nearest
    to the midpoint of the (N-k)-th and (N-k+1)-th smallest scores, so that exactly k
    scores exceed it when those two differ.  Returns float32 [H]."""
    e = np.asarray(e, dtype=np.float32)
    B, T, H = e.shape
    N = B * T
    k = int(round(rho * N))
    out = np.empty(H, dtype=np.float32)
    for h in range(H):
        if k == 0:
            out[h] = np.inf
        elif k == N:
            out[h] = -np.inf
        else:
            s = np.sort(e[:, :, h].reshape(-1).astype(np.float64))
            out[h] = np.float32(0.5 * (s[N - k - 1] + s[N - k]))
    return out


def route_stats(out, tau, near_band=1e-5):
    """Counts, KV usage rho and near-threshold counts from an oracle result.

    rho = sum of routed counts / (B*T*H) ([HAM] §5, KV-usage definition restricted
    to one layer); n_near[h] = number of tokens of head h with |e - tau| < near_band (tau per
    head [H] or per token and head [B,T,H]).
    """
    e = out["e"]
    B, T, H = e.shape
    routed = out["routed"].astype(np.int64)
    count = routed.sum(axis=1)                      # [B,H]
    rho = float(count.sum()) / float(B * T * H)
    tau = np.asarray(tau, dtype=np.float64)
    tau = tau.reshape(1, 1, H) if tau.size == H else tau.reshape(B, T, H)
    n_near = (np.abs(e - tau) < near_band).sum(axis=(0, 1))
    return dict(count=count, rho=rho, n_near=n_near)


def attention_backward(q_attn, Kc, Vc, pos, count, dO, *, scale, t0=0, doc_start=None):
    """Gradients of the attention readout ([HAM] §2 KV-memory equation; the visible
    set of App. A.1 "FlexAttention and Block Masks"), written out per head from the
    definition of softmax attention, in float64.  Query t (position t0 + t) sees the
    cached entries at positions <= t0 + t (and >= doc_start[b, t] if given).  With
    P = the masked softmax of scale * Q K^T (a row with no visible entry is 0),
    O = P V, D = rowsum(dO * O):  dP = dO V^T, dS = P * (dP - D),
    dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.  Returns dict(dq [B,T,H,dk],
    dKc [B,H,cap,dk], dVc [B,H,cap,dv]); cache rows >= count are 0."""
    q = np.asarray(q_attn, dtype=np.float64)
    B, T, H, dk = q.shape
    Kc = np.asarray(Kc, dtype=np.float64)
    Vc = np.asarray(Vc, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    cap, dv = Kc.shape[2], Vc.shape[3]
    dq = np.zeros((B, T, H, dk))
    dK = np.zeros((B, H, cap, dk))
    dV = np.zeros((B, H, cap, dv))
    tpos = t0 + np.arange(T)
    for b in range(B):
        for h in range(H):
            n = int(count[b, h])
            p_ = np.asarray(pos[b, h, :n], dtype=np.int64)
            vis = p_[None, :] <= tpos[:, None]
            if doc_start is not None:
                vis &= p_[None, :] >= np.asarray(doc_start[b], dtype=np.int64)[:, None]
            Q, K, V, G = q[b, :, h], Kc[b, h, :n], Vc[b, h, :n], dO[b, :, h]
            S = np.where(vis, scale * (Q @ K.T), -np.inf)
            P = np.zeros((T, n))
            rows = vis.any(axis=1)
            if rows.any():
                Sr = S[rows]
                E = np.exp(Sr - Sr.max(axis=1, keepdims=True))
                P[rows] = E / E.sum(axis=1, keepdims=True)
            O = P @ V
            D = (G * O).sum(axis=1, keepdims=True)
            dS = P * (G @ V.T - D)
            dq[b, :, h] = scale * dS @ K
            dK[b, h, :n] = scale * dS.T @ Q
            dV[b, h, :n] = P.T @ G
    return dict(dq=dq, dKc=dK, dVc=dV)


def rnn_backward(q, k, v, beta, g, dO, *, S0=None, dS_T=None):
    """Gradients of the gated delta-rule RNN readout ([HAM] §2 DeltaNet update and
    linear-attention readout, App. A.1 gated DeltaNet), written out per head in
    float64 by reverse-mode differentiation of the token-serial recurrence.

    Forward (per head):  p_t = S_{t-1}^T k_t,  r_t = v_t - alpha_t p_t,
    S_t = alpha_t S_{t-1} + beta_t k_t r_t^T,  o_t = S_t^T q_t,  alpha_t = exp(g_t).
    Given dO = dL/do_rnn [B,T,H,dv] and dS_T = dL/dS_T [B,H,dk,dv] (None: 0), with
    G = dL/dS_t accumulated from the end:
      G += q_t dO_t^T;  dq_t = S_t dO_t;  u_t = G^T k_t;
      dv_t = beta_t u_t;  dbeta_t = u_t . r_t;
      dk_t = beta_t (G r_t - alpha_t S_{t-1} u_t);
      dalpha_t = <G, S_{t-1}> - beta_t u_t . p_t;  dg_t = alpha_t dalpha_t;
      G <- alpha_t (G - beta_t k_t u_t^T)   (dL/dS_{t-1});   dS0 = G at the end.
    The routing decision passes no gradient (a hard threshold).  Returns dict(dq,
    dk [B,T,H,dk], dv [B,T,H,dv], dbeta, dg [B,T,H], dS0 [B,H,dk,dv])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    beta, g = np.asarray(beta, np.float64), np.asarray(g, np.float64)
    dO = np.asarray(dO, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = dict(dq=np.zeros((B, T, H, dk)), dk=np.zeros((B, T, H, dk)), dv=np.zeros((B, T, H, dv)),
               dbeta=np.zeros((B, T, H)), dg=np.zeros((B, T, H)), dS0=np.zeros((B, H, dk, dv)))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[b, h], dtype=np.float64)
            states = [S]                                   # S_{-1} = S0, then S_0 .. S_{T-1}
            for t in range(T):
                a = math.exp(g[b, t, h])
                p = S.T @ k[b, t, h]
                S = a * S + beta[b, t, h] * np.outer(k[b, t, h], v[b, t, h] - a * p)
                states.append(S)
            G = np.zeros((dk, dv)) if dS_T is None else np.array(dS_T[b, h], dtype=np.float64)
            for t in range(T - 1, -1, -1):
                a, bt = math.exp(g[b, t, h]), beta[b, t, h]
                kt, qt, vt, do = k[b, t, h], q[b, t, h], v[b, t, h], dO[b, t, h]
                Sp, St = states[t], states[t + 1]
                G = G + np.outer(qt, do)
                out["dq"][b, t, h] = St @ do
                p = Sp.T @ kt
                r = vt - a * p
                u = G.T @ kt
                out["dv"][b, t, h] = bt * u
                out["dbeta"][b, t, h] = u @ r
                out["dk"][b, t, h] = bt * (G @ r - a * (Sp @ u))
                out["dg"][b, t, h] = a * (np.sum(G * Sp) - bt * (u @ p))
                G = a * (G - bt * np.outer(kt, u))
            out["dS0"][b, h] = G
    return out

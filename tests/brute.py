"""Independent dense formulations used to pin the oracle (NumPy, fp64, tiny sizes).

None of this is the oracle's code path: the oracle walks tokens one by one; these
routines solve whole chunks with dense linear algebra or evaluate attention as
one masked softmax matrix.  Source: "Hybrid Associative Memories" (arXiv
2603.22325), §2 (KV memory, DeltaNet update, routing score) and App. A.1.
"""
from __future__ import annotations

import numpy as np
from scipy.special import softmax


def chunked_delta_rule(q, k, v, beta, g, S0=None, chunk=16):
    """Gated delta rule of one head solved chunk by chunk in closed form.

    Within a chunk with entering state S (d_k x d_v), log-decay cumsum G and
    strict-lower A[t,j] = exp(G_t - G_j) k_t.k_j, the write vectors D solve the
    unit lower-triangular system (I + diag(beta) A) D = diag(beta)(V - diag(e^G) K S)
    (numpy.linalg.solve).  Then
        readout    O  = diag(e^G) Q S + (Q K^T o Gamma o lower-incl) D
        prediction P  = diag(e^G) K S + A D        (P_t = alpha_t S_{t-1}^T k_t)
        next state S' = e^{G_C} S + sum_j e^{G_C - G_j} k_j D_j^T.
    Returns (O [T,dv], P [T,dv], S_T).
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    P = np.zeros((T, dv))
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(T, c0 + chunk))
        K, V, Q = k[sl], v[sl], q[sl]
        b = beta[sl]
        G = np.cumsum(g[sl])
        n = len(G)
        Gam = np.exp(G[:, None] - G[None, :])
        A = np.tril(K @ K.T * Gam, -1)
        D = np.linalg.solve(np.eye(n) + b[:, None] * A,
                            b[:, None] * (V - np.exp(G)[:, None] * (K @ S)))
        O[sl] = np.exp(G)[:, None] * (Q @ S) + np.tril(Q @ K.T * Gam) @ D
        P[sl] = np.exp(G)[:, None] * (K @ S) + A @ D
        S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ D
    return O, P, S


def masked_softmax_attention(q, k, v, allowed, scale):
    """o[t] = softmax over {j : allowed[t,j]} of scale*q_t.k_j applied to v; rows
    with no allowed key give 0.  One dense score matrix, scipy softmax."""
    s = scale * (q @ k.T)
    s = np.where(allowed, s, -np.inf)
    out = np.zeros((q.shape[0], v.shape[1]))
    rows = allowed.any(axis=1)
    if rows.any():
        p = softmax(s[rows], axis=1)
        out[rows] = p @ v
    return out


def cosine_distance_rows(p, v):
    """1 - cos(p_t, v_t) per row, with cos := 0 for a zero vector."""
    pv = (p * v).sum(1)
    npv = np.linalg.norm(p, axis=1) * np.linalg.norm(v, axis=1)
    c = np.where(npv > 0, pv / np.where(npv > 0, npv, 1.0), 0.0)
    return 1.0 - np.clip(c, -1.0, 1.0)

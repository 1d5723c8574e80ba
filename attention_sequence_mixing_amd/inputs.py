"""Seeded synthetic inputs for the HAM layer workloads.

This module holds no arithmetic of the method: it only draws random numbers,
shapes them like the inputs of one HAM sequence mixer, rounds them to the I/O
dtype, and picks a routing threshold from a given array of scores.  Both the
tests (on both sides of every comparison) and the benchmark use it.

Recipe (every workload): NumPy ``default_rng(seed)`` (PCG64); draws in the
fixed order q, k, v, beta_raw, g_raw, each in C order ``[B,T,H,d]`` or
``[B,T,H]``.  q and k ~ N(0,1) then L2-normalised over d per (b,t,h) in fp32;
v ~ N(0,1); beta = sigmoid(N(0,1)); g = -softplus(N(0,1)) (the log decay, so
alpha = exp(g) lies in (0,1)).  bf16 workloads round q, k, v to bf16
(round-to-nearest-even) after normalising; beta and g stay fp32.

The gated DeltaNet state of the "Hybrid Associative Memories" layer (§2,
App. A.1) needs beta*|k|^2 <= 2 for stability; unit keys and beta < 1 keep it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    d: int
    dtype: str            # "f32" or "bf16" (q, k, v, o and the cache)
    seed: int
    rho: float            # targeted KV usage
    scale: float = field(default=0.0)   # 0 -> 1/sqrt(d)
    needles: int = 0      # planted repeated (k, v) pairs per head

    @property
    def attn_scale(self) -> float:
        return self.scale if self.scale else 1.0 / math.sqrt(self.d)


# The workloads: a small fp32 case, the 800M-model-shape layer, a long-context
# case with planted repeated pairs, and the decode case (prefix + steps).
SMALL = Workload("small_f32_B1_H2_T256_d64", 1, 256, 2, 64, "f32", 0, 0.5, 1.0 / 8.0)
LAYER = Workload("layer_bf16_B8_H16_T4096_d128", 8, 4096, 16, 128, "bf16", 1, 0.5)
LONG = Workload("long_bf16_B1_H16_T32768_d128", 1, 32768, 16, 128, "bf16", 3, 0.25,
                needles=64)
DECODE_B, DECODE_H, DECODE_D, DECODE_PREFIX, DECODE_STEPS = 32, 16, 128, 32768, 256
RHO_SWEEP = (0.0, 0.1, 0.25, 0.5, 1.0)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    return (np.ascontiguousarray(x, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    x = x.astype(np.float32)
    n = np.sqrt((x * x).sum(axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _softplus(x):
    return np.logaddexp(0.0, x).astype(np.float32)


def make_inputs(B, T, H, dk, dv=None, *, dtype="f32", seed=0, needles=0):
    """Draw one batch of inputs.  Returns float32 numpy arrays (bf16-exact if dtype == 'bf16').

    q, k: [B,T,H,dk]; v: [B,T,H,dv]; beta, g: [B,T,H].
    needles > 0 plants that many (k*, v*) pairs per head, each written at two of
    2*needles distinct uniformly random positions shared across heads, over the
    N(0,1) background (k* unit, v* ~ N(0,1)).
    """
    dv = dk if dv is None else dv
    rng = np.random.default_rng(seed)
    q = _unit_rows(rng.standard_normal((B, T, H, dk), dtype=np.float32))
    k = _unit_rows(rng.standard_normal((B, T, H, dk), dtype=np.float32))
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    g = -_softplus(rng.standard_normal((B, T, H), dtype=np.float32))
    if needles:
        for b in range(B):
            where = rng.choice(T, size=2 * needles, replace=False)
            ks = _unit_rows(rng.standard_normal((needles, H, dk), dtype=np.float32))
            vs = rng.standard_normal((needles, H, dv), dtype=np.float32)
            for i in range(needles):
                for t in (where[2 * i], where[2 * i + 1]):
                    k[b, t] = ks[i]
                    v[b, t] = vs[i]
    if dtype == "bf16":
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return dict(q=q, k=k, v=v, beta=beta, g=g)


def make_workload(w: Workload):
    return make_inputs(w.B, w.T, w.H, w.d, dtype=w.dtype, seed=w.seed, needles=w.needles)


def tau_for_rho(e: np.ndarray, rho: float) -> np.ndarray:
    """Per-head threshold (float32, e-units) that routes round(rho*N) of the N = B*T
    scores of each head when there are no ties: the midpoint of the (N-k)-th and
    (N-k+1)-th smallest scores.  rho = 0 gives +inf, rho = 1 gives -inf."""
    e = np.asarray(e, dtype=np.float64)
    B, T, H = e.shape
    N = B * T
    kk = int(round(rho * N))
    tau = np.empty(H, dtype=np.float32)
    for h in range(H):
        if kk <= 0:
            tau[h] = np.inf
        elif kk >= N:
            tau[h] = -np.inf
        else:
            s = np.sort(e[:, :, h].reshape(-1))
            tau[h] = np.float32(0.5 * (s[N - kk - 1] + s[N - kk]))
    return tau


def make_router_scores(B, T, H, seed):
    """Synthetic learned-router scores [B,T,H] float32 in (0, 1): sigmoid(N(0,1)) per
    token and head, standing in for sigma(W_r x_t) of a trained input router (no
    weights exist for it here)."""
    rng = np.random.default_rng(seed + 500)
    return _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))


def make_gates(B, T, H, seed):
    """Optional per-(t,h) mixing gates in (0,1), drawn as sigmoid(N(0,1))."""
    rng = np.random.default_rng(seed + 1000)
    gr = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    gk = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    return gr, gk


def doc_start_from_lengths(lengths, t0=0):
    """[T] int32 absolute start position of each token's document for one packed
    sequence made of documents of the given lengths, beginning at position t0."""
    out, s = [], t0
    for n in lengths:
        out.append(np.full(int(n), s, np.int32))
        s += int(n)
    return np.concatenate(out) if out else np.zeros(0, np.int32)


def make_doc_lengths(T, mean_len, seed):
    """Document lengths of one packed sequence of T tokens: geometric lengths with
    the given mean (at least 1), the last document cut to fill T exactly."""
    rng = np.random.default_rng(seed + 2000)
    lengths, left = [], T
    while left > 0:
        n = min(left, int(rng.geometric(1.0 / max(mean_len, 1.0))))
        lengths.append(n)
        left -= n
    return lengths


def make_doc_start(B, T, mean_len, seed, t0=0):
    """[B,T] int32 document starts of B packed sequences (geometric lengths)."""
    return np.stack([doc_start_from_lengths(make_doc_lengths(T, mean_len, seed + 7 * b), t0)
                     for b in range(B)])


def make_inputs_torch(B, T, H, dk, dv=None, *, dtype="bf16", seed=0, device="cuda"):
    """The same recipe drawn on the device with torch's generator (for workloads too
    large to draw on the host, e.g. a 32K-token prefix of 32 sequences).  Deterministic
    for a given device and torch build; not bit-identical to make_inputs."""
    import torch
    dv = dk if dv is None else dv
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def unit(shape):
        x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        x /= x.norm(dim=-1, keepdim=True)
        return x.to(tdt)

    q = unit((B, T, H, dk))
    k = unit((B, T, H, dk))
    v = torch.randn((B, T, H, dv), generator=gen, device=device, dtype=torch.float32).to(tdt)
    beta = torch.sigmoid(torch.randn((B, T, H), generator=gen, device=device))
    g = -torch.nn.functional.softplus(torch.randn((B, T, H), generator=gen, device=device))
    return dict(q=q, k=k, v=v, beta=beta.contiguous(), g=g.contiguous())

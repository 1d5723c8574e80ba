"""GPU test of ham_decode_step_noalloc, the decode step whose scratch is the
library's fixed per-GPU array (for callers that cannot allocate device memory).

It runs the same kernels as ham_decode_step with a caller workspace; two calls in a
row, the second on a smaller problem (fewer sequences and heads, smaller heads and
cache), must give exactly what ham_decode_step gives on copies of the same state and
cache.  A step needing more scratch than the array holds is rejected before
anything is enqueued, and the state is left untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd import _lib
from attention_sequence_mixing_amd.inputs import make_inputs, tau_for_rho
import oracle
from parity import to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _prefilled(B, T0, H, d, dtype, seed):
    """A cache and state from a forward over T0 tokens, and the next token's inputs."""
    inp = make_inputs(B, T0 + 1, H, d, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    e = oracle.forward(**{n: a[:, :T0] for n, a in inp.items()}, tau=np.full(H, np.inf, np.float32),
                       scale=d ** -0.5)["e"]
    tau = torch.from_numpy(tau_for_rho(e, 0.5)).to(DEV)
    t = to_dev(inp, dtype, DEV)
    pre = {n: x[:, :T0].contiguous() for n, x in t.items()}
    out = ham.ham_forward(pre["q"], pre["k"], pre["v"], pre["beta"], pre["g"], tau, scale=d ** -0.5,
                          cap=T0 + 8)
    torch.cuda.synchronize()
    x = {n: t[n][:, T0].contiguous() for n in t}
    return x, tau, out


def _step(plan, x, tau, out, T0):
    S = out["S"].clone()
    cache = {n: out[n].clone() for n in ("Kc", "Vc", "pos", "count")}
    B = S.shape[0]
    plan(x["q"], x["k"], x["v"], x["beta"], x["g"], tau, S, cache["Kc"], cache["Vc"], cache["pos"],
         cache["count"], torch.full((B,), T0, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    return dict(o=plan.o.clone(), o_rnn=plan.o_rnn.clone(), e=plan.e.clone(), routed=plan.routed.clone(),
                S=S, **cache)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_decode_equals_workspace_decode(dtype):
    # larger problem first, then a smaller one: the second call reuses the array the
    # first one left behind
    for (B, T0, H, d, seed) in ((4, 1500, 3, 128, 400), (2, 200, 2, 64, 401)):
        print(f"noalloc decode: dtype={dtype} B={B} prefix={T0} H={H} d={d}", flush=True)
        x, tau, out = _prefilled(B, T0, H, d, dtype, seed)
        ref_plan = ham.DecodePlan(B, H, d, d, T0 + 8, dtype, DEV, want_o_rnn=True)
        na_plan = ham.DecodePlan(B, H, d, d, T0 + 8, dtype, DEV, want_o_rnn=True, noalloc=True)
        assert na_plan.ws is None
        ref = _step(ref_plan, x, tau, out, T0)
        got = _step(na_plan, x, tau, out, T0)
        for n in ref:
            assert torch.equal(ref[n], got[n]), (n, B, H, d)


def test_noalloc_rejects_steps_beyond_its_array():
    """A cache so long that the split-K partials exceed the array: HAM_EWORKSPACE, and
    nothing runs (the state and count stay as they were)."""
    L = _lib.lib()
    limit = L.ham_decode_noalloc_scratch_bytes()
    assert limit == 32 << 20
    B, H, d = 16, 16, 128
    cap = 1 << 22
    dims = ham.make_dims(B, 1, H, d, d, _lib.HAM_BF16, d ** -0.5, 1e-6, cap)
    assert L.ham_decode_workspace_size(ctypes.byref(dims)) > limit
    plan = ham.DecodePlan(B, H, d, d, 8, torch.bfloat16, DEV, noalloc=True)
    plan.dims.cap = cap                       # the same plan at a far larger capacity
    x = {n: torch.zeros((B, H, d), dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    sc = {n: torch.zeros((B, H), dtype=torch.float32, device=DEV) for n in ("beta", "g")}
    S = torch.ones((B, H, d, d), dtype=torch.float32, device=DEV)
    Kc = torch.zeros((B, H, 8, d), dtype=torch.bfloat16, device=DEV)
    pos = torch.zeros((B, H, 8), dtype=torch.int32, device=DEV)
    count = torch.zeros((B, H), dtype=torch.int32, device=DEV)
    tau = torch.zeros((H,), dtype=torch.float32, device=DEV)
    t_abs = torch.zeros((B,), dtype=torch.int32, device=DEV)
    args = [ctypes.byref(plan.dims)] + [ctypes.c_void_p(p.data_ptr()) for p in
                                        (x["q"], x["k"], x["v"])] + [None] * 3 + \
        [ctypes.c_void_p(p.data_ptr()) for p in (sc["beta"], sc["g"], tau)] + [None] * 4 + \
        [ctypes.c_void_p(p.data_ptr()) for p in (S, Kc, Kc, pos, count, t_abs, plan.o)] + [None] * 2 + \
        [ctypes.c_void_p(plan.e.data_ptr()), ctypes.c_void_p(plan.routed.data_ptr()), None, None]
    rc = L.ham_decode_step_noalloc(*args)
    assert rc == _lib.HAM_EWORKSPACE
    assert "more than" in L.ham_last_error().decode()
    torch.cuda.synchronize()
    assert torch.all(S == 1.0) and torch.all(count == 0)

"""GPU parity of the gated delta-rule RNN gradients (ham_rnn_backward) against the
oracle's reverse-mode derivatives of the token-serial recurrence ("Hybrid Associative
Memories" §2 DeltaNet update and readout, App. A.1 gated DeltaNet; the pages train the
layer end to end).  Every gradient (q, k, v, beta, g and the entering state) per (b,h)
slice within 1e-4 of the slice's largest value: the kernel computes in fp32 from
the same input values the oracle reads."""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import LAYER, make_inputs, make_workload
from parity import np_of, rel_err_slices, to_dev

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 1e-4


def _rel(x, y, axes):
    return rel_err_slices(x, y, axes)


@pytest.mark.parametrize("recurrent", [False, True], ids=["chunked", "token_serial"])
@pytest.mark.parametrize("B,T,H,dk,dv,dtype,s0,dst", [
    (2, 37, 2, 64, 64, torch.float32, False, False),
    (1, 130, 3, 128, 128, torch.bfloat16, True, True),
    (2, 65, 1, 64, 128, torch.float32, True, False),
    (1, 200, 2, 128, 64, torch.bfloat16, False, True),
    (1, 1, 2, 128, 128, torch.float32, True, True),
    (1, 64, 1, 64, 64, torch.float32, True, True),
    (1, 128, 2, 128, 128, torch.float32, False, True),
    (2, 1024, 2, 128, 128, torch.bfloat16, True, True),
])
def test_rnn_backward(B, T, H, dk, dv, dtype, s0, dst, recurrent):
    seed = 500 + T + dk
    inp = make_inputs(B, T, H, dk, dv, dtype="f32" if dtype == torch.float32 else "bf16", seed=seed)
    rng = np.random.default_rng(seed)
    S0 = (0.3 * rng.standard_normal((B, H, dk, dv))).astype(np.float32) if s0 else None
    dO = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    dS_T = rng.standard_normal((B, H, dk, dv)).astype(np.float32) if dst else None
    t = to_dev(inp, dtype, DEV)
    dev = lambda x: None if x is None else torch.from_numpy(x).to(DEV)
    print(f"rnn backward ({'token-serial' if recurrent else 'chunked'}): B={B} T={T} H={H} {dk}/{dv} {dtype} "
          f"S0={s0} dS_T={dst}", flush=True)
    got = ham.ham_rnn_backward(t["q"], t["k"], t["v"], t["beta"], t["g"], dev(dO), S0=dev(S0), dS_T=dev(dS_T),
                               force_recurrent=recurrent)
    torch.cuda.synchronize()
    ref = oracle.rnn_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["g"], dO, S0=S0, dS_T=dS_T)
    errs = {n: _rel(np_of(got[n]), ref[n], 2) for n in ("dq", "dk", "dv")}
    errs.update({n: _rel(np_of(got[n])[..., None], ref[n][..., None], 2) for n in ("dbeta", "dg")})
    errs["dS0"] = _rel(np_of(got["dS0"]), ref["dS0"], 1)
    print("   errors", {k: f"{v:.2e}" for k, v in errs.items()})
    assert all(v < TOL for v in errs.values()), errs


def test_rnn_backward_layer_shape_sampled_heads():
    """The chunked gradients at the headline layer shape (B 8, T 4096, H 16, d 128, bf16
    inputs, dO and dS_T ~ N(0,1)), every head computed on the GPU; three (b, h) slices
    compared with the oracle, which runs on those slices alone (heads are independent)."""
    w = LAYER
    inp = make_workload(w)
    rng = np.random.default_rng(77)
    dO = rng.standard_normal((w.B, w.T, w.H, w.d)).astype(np.float32)
    dS_T = rng.standard_normal((w.B, w.H, w.d, w.d)).astype(np.float32)
    t = to_dev(inp, torch.bfloat16, DEV)
    print(f"rnn backward at the layer shape: B={w.B} T={w.T} H={w.H} d={w.d}", flush=True)
    got = ham.ham_rnn_backward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(dO).to(DEV),
                               dS_T=torch.from_numpy(dS_T).to(DEV))
    torch.cuda.synchronize()
    got = {n: np_of(x) for n, x in got.items()}
    for b, h in [(0, 0), (3, 7), (7, 15)]:
        sl = lambda x: np.ascontiguousarray(x[b:b + 1, :, h:h + 1])
        ref = oracle.rnn_backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["g"]),
                                  sl(dO), dS_T=np.ascontiguousarray(dS_T[b:b + 1, h:h + 1]))
        errs = {n: _rel(sl(got[n]), ref[n], 2) for n in ("dq", "dk", "dv")}
        errs.update({n: _rel(sl(got[n])[..., None], ref[n][..., None], 2) for n in ("dbeta", "dg")})
        errs["dS0"] = _rel(got["dS0"][b:b + 1, h:h + 1], ref["dS0"], 1)
        print(f"   (b, h) = ({b}, {h}) errors", {k: f"{v:.2e}" for k, v in errs.items()}, flush=True)
        assert all(v < TOL for v in errs.values()), (b, h, errs)


def test_rnn_backward_rejects_other_head_sizes():
    q = torch.zeros((1, 8, 1, 256), dtype=torch.bfloat16, device=DEV)
    v = torch.zeros((1, 8, 1, 384), dtype=torch.bfloat16, device=DEV)
    s = torch.zeros((1, 8, 1), dtype=torch.float32, device=DEV)
    with pytest.raises(ham.HamError):
        ham.ham_rnn_backward(q, q, v, s, s, torch.zeros((1, 8, 1, 384), device=DEV))

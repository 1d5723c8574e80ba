"""GPU parity of the segmented chunked state pass.

With few heads (B*H*dv/64 workgroups of the state pass filling at most half the
CUs) and long sequences, the library cuts the chunk sequence into segments: each
segment's zero-start state B_p and transition A_p (the same pass with V = 0 from
S = I) are formed side by side, the entering states follow from S_in[p+1] = A_p
S_in[p] + B_p, and the full pass then runs every segment from its entering state.
The result is the same recurrence ("Hybrid Associative Memories" §2, App. A.1),
reassociated; it is compared with the token-serial oracle like the one-segment path.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, make_gates, tau_for_rho
from parity import check_forward, check_routing, np_of, rel_err_slices, to_dev, TOL

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
INF = np.float32(np.inf)


def _tau(inp, rho, scale):
    e = oracle.forward(**inp, tau=np.full(inp["q"].shape[2], INF, np.float32), scale=scale)["e"]
    return tau_for_rho(e, rho)


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 2600, 2, 128, 128), (1, 1100, 1, 64, 128),
                                         (1, 1600, 2, 128, 64), (2, 1333, 1, 64, 64),
                                         (1, 4160, 3, 128, 128)])
def test_segmented_forward(B, T, H, dk, dv):
    seed = 160 + T
    inp = make_inputs(B, T, H, dk, dv, dtype="bf16", seed=seed)
    scale = dk ** -0.5
    tau = _tau(inp, 0.3, scale)
    gr, gk = make_gates(B, T, H, seed)
    t = to_dev(inp, torch.bfloat16, DEV)
    out = ham.ham_forward(t["q"], t["k"], t["v"], t["beta"], t["g"], torch.from_numpy(tau).to(DEV),
                          scale=scale, gate_rnn=torch.from_numpy(gr).to(DEV),
                          gate_kv=torch.from_numpy(gk).to(DEV), want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    res = check_forward(out, inp, tau, torch.bfloat16, scale=scale, gates=(gr, gk))
    print(f"segmented B{B} T{T} H{H} {dk}/{dv}: errors {res['errs']} near-band flips {res['nflip']}")


def test_segmented_continuation_and_route_stats():
    """A continued call (entering state S0 and an existing cache) on the segmented
    path, and the routing-only entry point on it."""
    B, T, H, d = 1, 3000, 2, 128
    T1 = 1200
    inp = make_inputs(B, T, H, d, dtype="bf16", seed=170)
    scale = d ** -0.5
    tau = _tau(inp, 0.4, scale)
    first = {n: a[:, :T1] for n, a in inp.items()}
    second = {n: a[:, T1:] for n, a in inp.items()}
    t1, t2 = to_dev(first, torch.bfloat16, DEV), to_dev(second, torch.bfloat16, DEV)
    tau_d = torch.from_numpy(tau).to(DEV)
    o1 = ham.ham_forward(t1["q"], t1["k"], t1["v"], t1["beta"], t1["g"], tau_d, scale=scale, cap=T)
    cache = {n: o1[n] for n in ("Kc", "Vc", "pos", "count")}
    o2 = ham.ham_forward(t2["q"], t2["k"], t2["v"], t2["beta"], t2["g"], tau_d, scale=scale,
                         S0=o1["S"].clone(), cache=cache, t0=T1, want_o_rnn=True, want_o_kv=True)
    torch.cuda.synchronize()
    ref1 = oracle.forward(**first, tau=tau, scale=scale, cap=T)
    ref_cache = {n: ref1[n] for n in ("Kc", "Vc", "pos", "count")}
    check_routing(o1["e"].cpu().numpy(), o1["routed"].cpu().numpy(), ref1, tau)
    check_forward(o2, second, tau, torch.bfloat16, scale=scale, S0=ref1["S"], cache=ref_cache, t0=T1)
    t = to_dev(inp, torch.bfloat16, DEV)
    st = ham.ham_route_stats(t["k"], t["v"], t["beta"], t["g"], tau_d)
    ref = oracle.forward(**inp, tau=tau, scale=scale, emit=np.zeros((B, T, H), np.int8))
    check_routing(st["e"].cpu().numpy(), st["routed"].cpu().numpy(), ref, tau)
    assert np.array_equal(st["count"].cpu().numpy(), st["routed"].cpu().numpy().sum(axis=1))

"""GPU parity of the attention gradients (training; "Hybrid Associative Memories" §2
KV-memory equation, the visible set of App. A.1).

The cache (Kc, Vc, pos, count) comes from the oracle's forward with a fixed routing
mask, so both sides differentiate the same readout; the GPU kernels get it converted
to the io dtype.  dq, dKc and dVc (fp32) are compared with the oracle's backward,
written from the definition of softmax attention and pinned by finite differences.
Cases: both io dtypes, the four head-size pairs, ragged T, document masks, a cache
continued from an earlier call, and queries that see no entry.
"""
import numpy as np
import pytest
import torch

import oracle
import attention_sequence_mixing_amd as ham
from attention_sequence_mixing_amd.inputs import make_inputs, make_doc_start, bf16_round
from parity import np_of, rel_err_slices

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-4, torch.bfloat16: 1e-3}


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).to(DEV)


@pytest.mark.parametrize("B,T,H,dk,dv,t1,docs", [
    (2, 150, 2, 64, 64, 0, False),
    (1, 200, 3, 128, 128, 0, True),
    (2, 97, 2, 64, 128, 40, False),
    (1, 130, 2, 128, 64, 60, True),
    (1, 700, 2, 128, 128, 0, False),                  # several 64-query and 64-entry tiles
    (2, 451, 2, 64, 128, 90, True),
])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_attention_backward(B, T, H, dk, dv, t1, docs, dtype):
    dt = "f32" if dtype == torch.float32 else "bf16"
    seed = 220 + T + dk
    inp = make_inputs(B, T, H, dk, dv, dtype=dt, seed=seed)
    att = make_inputs(B, T, H, dk, dv, dtype=dt, seed=seed + 1)
    rng = np.random.default_rng(seed)
    mask = (rng.random((B, T, H)) < 0.4).astype(np.int8)
    mask[:, :3] = 0                                   # the first queries see nothing
    ds = make_doc_start(B, T, 30, seed) if docs else None
    scale = dk ** -0.5
    # the cache of an earlier call (t1 tokens), then this call's T - t1 tokens
    kw = dict(tau=np.zeros(H, np.float32), scale=scale, cap=T)
    first = oracle.forward(**{n: x[:, :t1 or 1] for n, x in inp.items()}, mask_override=mask[:, :t1 or 1],
                           q_attn=att["q"][:, :t1 or 1], k_attn=att["k"][:, :t1 or 1],
                           v_attn=att["v"][:, :t1 or 1], **kw) if t1 else None
    cur = {n: x[:, t1:] for n, x in inp.items()}
    ref = oracle.forward(**cur, mask_override=mask[:, t1:], q_attn=att["q"][:, t1:], k_attn=att["k"][:, t1:],
                         v_attn=att["v"][:, t1:], t0=t1, S0=None if first is None else first["S"],
                         cache=None if first is None else {n: first[n] for n in ("Kc", "Vc", "pos", "count")},
                         doc_start=None if ds is None else ds[:, t1:], **kw)
    Tc = T - t1
    dO = rng.standard_normal((B, Tc, H, dv)).astype(np.float32)
    want = oracle.attention_backward(att["q"][:, t1:], ref["Kc"], ref["Vc"], ref["pos"], ref["count"], dO,
                                     scale=scale, t0=t1, doc_start=None if ds is None else ds[:, t1:])
    cache = dict(Kc=_dev(ref["Kc"], dtype), Vc=_dev(ref["Vc"], dtype),
                 pos=torch.from_numpy(ref["pos"].astype(np.int32)).to(DEV),
                 count=torch.from_numpy(ref["count"].astype(np.int32)).to(DEV))
    got = ham.ham_attention_backward(_dev(att["q"][:, t1:], dtype), cache, torch.from_numpy(dO).to(DEV),
                                     scale=scale, t0=t1,
                                     doc_start=None if ds is None else
                                     torch.from_numpy(ds[:, t1:].astype(np.int32)).to(DEV))
    torch.cuda.synchronize()
    tol = TOL[dtype]
    assert rel_err_slices(np_of(got["dq"]), want["dq"], 2) < tol
    cnt = ref["count"]
    for b in range(B):
        for h in range(H):
            n = int(cnt[b, h])
            for name in ("dKc", "dVc"):
                x, y = np_of(got[name][b, h, :n]), want[name][b, h, :n]
                assert np.abs(x - y).max() <= tol * max(np.abs(y).max(), 1e-30), (name, b, h)
    assert np.abs(np_of(got["dq"][:, :3])).max() == 0 if t1 == 0 else True


def test_attention_backward_rejects_what_it_does_not_cover():
    B, T, H, d = 1, 8, 1, 64
    q = torch.zeros((B, T, H, d), device=DEV)
    cache = dict(Kc=torch.zeros((B, H, T, d), device=DEV), Vc=torch.zeros((B, H, T, d), device=DEV),
                 pos=torch.zeros((B, H, T), dtype=torch.int32, device=DEV),
                 count=torch.zeros((B, H), dtype=torch.int32, device=DEV))
    from attention_sequence_mixing_amd import _lib, make_dims
    import ctypes
    L = _lib.lib()
    for kw in (dict(rope_base=10000.0), dict(route_block=4)):
        dims = make_dims(B, T, H, d, d, 0, 0.125, 1e-6, T, **kw)
        assert L.ham_attention_backward(ctypes.byref(dims), *([ctypes.c_void_p(q.data_ptr())] * 10),
                                        ctypes.c_void_p(q.data_ptr()), 1 << 20, None) == _lib.HAM_EUNSUPPORTED

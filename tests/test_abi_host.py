"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol that include/ham.h declares, sizes its workspaces and rejects bad arguments
before enqueuing anything."""
import ctypes
import os
import re

import pytest

from attention_sequence_mixing_amd import _lib
from attention_sequence_mixing_amd._lib import HamDims

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "ham.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ham_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    L = _lib.lib()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert L.ham_version() >= 10000


def dims(**kw):
    d = dict(B=2, T=300, H=4, dk=128, dv=128, io_dtype=1, scale=0.088, norm_eps=1e-6, cap=300,
             flags=0, t0=0)
    d.update(kw)
    return HamDims(**d)


def test_workspace_sizes():
    L = _lib.lib()
    d = dims()
    ws = L.ham_forward_workspace_size(ctypes.byref(d))
    BTH = 2 * 300 * 4
    assert ws >= BTH * 128 * 4 + BTH * 4 + BTH      # o_rnn fp32 + e + routed at least
    assert L.ham_route_stats_workspace_size(ctypes.byref(d)) > ws   # adds the state
    assert L.ham_decode_workspace_size(ctypes.byref(d)) > 0
    # the paper's layer: RNN heads 256/384 with twice as many KV heads of 128/192
    assert L.ham_forward_workspace_size(ctypes.byref(dims(dk=256, dv=384, kv_heads=8, dk_kv=128,
                                                          dv_kv=192))) > 0
    for bad in (dims(dk=96), dims(dv=32), dims(dk=256), dims(dv=384), dims(dk=256, dv=384),
                dims(T=0), dims(B=-1),
                dims(io_dtype=7), dims(cap=0), dims(flags=64), dims(dk_kv=128, dv_kv=192)):
        assert L.ham_forward_workspace_size(ctypes.byref(bad)) == 0


def test_rope_workspace_and_base_checks():
    """A rotary base adds one table of T x dk/2 (cos, sin) float pairs to the forward
    workspace; a negative, infinite or NaN base is rejected."""
    L = _lib.lib()
    ws0 = L.ham_forward_workspace_size(ctypes.byref(dims()))
    ws1 = L.ham_forward_workspace_size(ctypes.byref(dims(rope_base=500000.0)))
    assert ws1 - ws0 >= 300 * 64 * 8
    assert L.ham_decode_workspace_size(ctypes.byref(dims(rope_base=10000.0))) > 0
    for bad in (-1.0, float("nan"), float("inf")):
        for fn in (L.ham_forward_workspace_size, L.ham_decode_workspace_size):
            assert fn(ctypes.byref(dims(rope_base=bad))) == 0
            assert "rope_base" in _msg()


def _fwd(d, ptrs=None, ws_bytes=1 << 40):
    P = ctypes.c_void_p
    fake = P(1 << 20)   # an aligned non-NULL host value; never dereferenced by these checks
    args = [fake] * 24 if ptrs is None else ptrs
    return _lib.lib().ham_forward(ctypes.byref(d), *args, ws_bytes, None)


def _msg():
    return _lib.lib().ham_last_error().decode()


def test_forward_argument_errors():
    P = ctypes.c_void_p
    fake = P(1 << 20)
    base = [fake] * 24
    # dims
    assert _fwd(dims(dk=100)) == _lib.HAM_EUNSUPPORTED
    assert "dk" in _msg()
    assert _fwd(dims(B=0)) == _lib.HAM_EINVAL
    assert _fwd(dims(io_dtype=3)) == _lib.HAM_EUNSUPPORTED
    assert _fwd(dims(flags=32)) == _lib.HAM_EUNSUPPORTED
    assert _fwd(dims(scale=0.0)) == _lib.HAM_EINVAL and "scale" in _msg()
    assert _fwd(dims(scale=-1.0)) == _lib.HAM_EINVAL
    # required pointers: q k v (0-2), beta g tau (6-8), S_out (13), o (14), Kc Vc pos count (19-22)
    for i in (0, 1, 2, 6, 7, 8, 13, 14, 19, 20, 21, 22):
        a = list(base)
        a[i] = None
        assert _fwd(dims(), a) == _lib.HAM_EINVAL, i
        assert "NULL" in _msg()
    # misaligned
    a = list(base)
    a[0] = P((1 << 20) + 2)
    assert _fwd(dims(), a) == _lib.HAM_EINVAL and "aligned" in _msg()
    assert _fwd(dims(cap=(1 << 22) + 1)) == _lib.HAM_EUNSUPPORTED and "cap" in _msg()
    assert _fwd(dims(T=0)) == _lib.HAM_EINVAL
    # capacity without continuation
    assert _fwd(dims(cap=100)) == _lib.HAM_ECAPACITY
    # workspace
    a = list(base)
    a[23] = None
    assert _fwd(dims(), a) == _lib.HAM_EWORKSPACE
    assert _fwd(dims(), base, ws_bytes=16) == _lib.HAM_EWORKSPACE


def test_decode_and_stats_argument_errors():
    L = _lib.lib()
    P = ctypes.c_void_p
    fake = P(1 << 20)
    a = [fake] * 26
    a[17] = None                                       # count
    assert L.ham_decode_step(ctypes.byref(dims()), *a, 1 << 40, None) == _lib.HAM_EINVAL
    a = [fake] * 26
    a[18] = None                                       # t_abs
    assert L.ham_decode_step(ctypes.byref(dims()), *a, 1 << 40, None) == _lib.HAM_EINVAL
    a = [fake] * 26
    assert L.ham_decode_step(ctypes.byref(dims()), *a, 8, None) == _lib.HAM_EWORKSPACE
    s = [fake] * 11
    s[9] = None                                        # count
    assert L.ham_route_stats(ctypes.byref(dims()), *s, ctypes.c_float(1e-5), None, fake,
                             1 << 40, None) == _lib.HAM_EINVAL
    s = [fake] * 11
    assert L.ham_route_stats(ctypes.byref(dims()), *s, ctypes.c_float(-1.0), None, fake,
                             1 << 40, None) == _lib.HAM_EINVAL


def test_product_path_has_no_oracle_dependency():
    """The library and binding never reference the oracle."""
    pkg = os.path.join(ROOT, "attention_sequence_mixing_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower(), f
    with open(_lib.LIB_PATH, "rb") as fh:
        assert b"ham_oracle" not in fh.read()


def test_select_tau_and_external_score_errors():
    L = _lib.lib()
    P = ctypes.c_void_p
    fake = P(1 << 20)
    d = dims(B=2, T=100, H=3)
    assert L.ham_select_tau(ctypes.byref(d), fake, ctypes.c_double(1.5), fake, None) == _lib.HAM_EINVAL
    assert "rho" in _msg()
    assert L.ham_select_tau(ctypes.byref(d), fake, ctypes.c_double(float("nan")), fake, None) == _lib.HAM_EINVAL
    assert L.ham_select_tau(ctypes.byref(d), None, ctypes.c_double(0.5), fake, None) == _lib.HAM_EINVAL
    assert L.ham_select_tau(ctypes.byref(dims(B=0)), fake, ctypes.c_double(0.5), fake, None) == _lib.HAM_EINVAL
    assert L.ham_select_tau(ctypes.byref(dims(B=65536, T=65536)), fake, ctypes.c_double(0.5), fake,
                            None) == _lib.HAM_EINVAL
    # external scores need e
    base = [fake] * 24
    a = list(base)
    a[17] = None                                       # e
    assert _fwd(dims(flags=_lib.HAM_EXTERNAL_SCORES), a) == _lib.HAM_EINVAL and "EXTERNAL" in _msg()
    a = [fake] * 26
    a[22] = None                                       # e of the decode step
    assert L.ham_decode_step(ctypes.byref(dims(flags=_lib.HAM_EXTERNAL_SCORES)), *a, 1 << 40, None) == _lib.HAM_EINVAL
    s = [fake] * 11
    assert L.ham_route_stats(ctypes.byref(dims(flags=_lib.HAM_EXTERNAL_SCORES)), *s, ctypes.c_float(1e-5), None,
                             fake, 1 << 40, None) == _lib.HAM_EUNSUPPORTED


def test_route_block_checks():
    """Block-contiguous routing: the block size is 0, 1 or a power of two up to 64;
    a forward (and route_stats) call covers whole blocks; the decode step needs the
    open blocks' score sums; route_stats does not count near-threshold tokens then."""
    L = _lib.lib()
    P = ctypes.c_void_p
    fake = P(1 << 20)
    for bad in (3, 12, 128, -1):
        assert L.ham_forward_workspace_size(ctypes.byref(dims(route_block=bad))) == 0
        assert "route_block" in _msg()
        assert _fwd(dims(route_block=bad)) == _lib.HAM_EUNSUPPORTED
    for ok in (0, 1, 2, 4, 16, 64):
        assert L.ham_forward_workspace_size(ctypes.byref(dims(T=320, cap=320, route_block=ok))) > 0
    assert _fwd(dims(T=300, route_block=16)) == _lib.HAM_EINVAL and "multiples" in _msg()
    assert _fwd(dims(T=320, cap=320, t0=8, route_block=16)) == _lib.HAM_EINVAL
    a = [fake] * 26
    a[12] = None                                       # block_score
    assert L.ham_decode_step(ctypes.byref(dims(route_block=16)), *a, 1 << 40, None) == _lib.HAM_EINVAL
    assert "block_score" in _msg()
    s = [fake] * 11
    assert L.ham_route_stats(ctypes.byref(dims(T=320, cap=320, route_block=16)), *s, ctypes.c_float(1e-5),
                             None, fake, 1 << 40, None) == _lib.HAM_EUNSUPPORTED


def test_kv_head_geometry_checks():
    """Attention heads of their own geometry: a multiple of H, sizes 64 or 128, value
    columns tiling the RNN heads' output, and their own q/k/v inputs."""
    L = _lib.lib()
    fake = ctypes.c_void_p(1 << 20)
    assert L.ham_forward_workspace_size(ctypes.byref(dims(kv_heads=8, dv_kv=64))) > 0
    assert L.ham_forward_workspace_size(ctypes.byref(dims(kv_heads=8, dv_kv=64))) > \
        L.ham_forward_workspace_size(ctypes.byref(dims()))           # the readout scratch
    assert L.ham_decode_workspace_size(ctypes.byref(dims(kv_heads=8, dk_kv=64, dv_kv=64))) > 0
    for bad, code in ((dims(kv_heads=6, dv_kv=64), _lib.HAM_EUNSUPPORTED),     # not a multiple of H
                      # values tile the RNN heads, but only two KV heads per RNN head are mixed
                      (dims(H=5, dk=256, dv=384, kv_heads=15, dk_kv=128, dv_kv=128), _lib.HAM_EUNSUPPORTED),
                      (dims(H=5, dk=256, dv=384, kv_heads=30, dk_kv=64, dv_kv=64), _lib.HAM_EUNSUPPORTED),
                      (dims(kv_heads=16, dk_kv=64, dv_kv=32), _lib.HAM_EUNSUPPORTED),
                      (dims(kv_heads=8), _lib.HAM_EUNSUPPORTED),               # 8*128 != 4*128
                      (dims(dk_kv=96), _lib.HAM_EUNSUPPORTED),
                      (dims(kv_heads=-1), _lib.HAM_EINVAL)):
        assert L.ham_forward_workspace_size(ctypes.byref(bad)) == 0
        assert _fwd(bad) == code
    a = [fake] * 24
    a[3] = None                                        # q_attn
    assert _fwd(dims(kv_heads=8, dv_kv=64), a) == _lib.HAM_EINVAL and "q_attn" in _msg()
    assert _fwd(dims(dk_kv=64), a) == _lib.HAM_EINVAL
    d = [fake] * 26
    d[5] = None                                        # v_attn of the decode step
    assert L.ham_decode_step(ctypes.byref(dims(kv_heads=8, dv_kv=64)), *d, 1 << 40, None) == _lib.HAM_EINVAL


def test_route_stats_ignores_the_kv_geometry():
    """Routing alone needs no attention heads: the paper's RNN heads (256/384) size a
    route-statistics workspace without KV sizes, while a forward needs them."""
    L = _lib.lib()
    d = dims(dk=256, dv=384)
    assert L.ham_route_stats_workspace_size(ctypes.byref(d)) > 0
    assert L.ham_forward_workspace_size(ctypes.byref(d)) == 0 and "dk_kv" in _msg()

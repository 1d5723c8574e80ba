"""ctypes view of libham.so (the C ABI of include/ham.h).

Loading fails loudly when the library has not been built: there is no fallback
path of any kind.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libham.so")

HAM_OK, HAM_EINVAL, HAM_EUNSUPPORTED, HAM_ECAPACITY, HAM_EHIP, HAM_EWORKSPACE = 0, -1, -2, -3, -4, -5
HAM_F32, HAM_BF16 = 0, 1
HAM_CONTINUE, HAM_FORCE_RECURRENT, HAM_EXTERNAL_SCORES, HAM_TAU_PER_TOKEN, HAM_OVERLAP = 1, 2, 4, 8, 16

# every symbol include/ham.h declares
EXPORTS = ("ham_version", "ham_last_error", "ham_forward_workspace_size", "ham_forward",
           "ham_decode_workspace_size", "ham_decode_step", "ham_route_stats_workspace_size",
           "ham_route_stats", "ham_select_tau", "ham_profile_start", "ham_profile_stop",
           "ham_attention_backward_workspace_size", "ham_attention_backward",
           "ham_decode_step_noalloc", "ham_decode_noalloc_scratch_bytes",
           "ham_rnn_backward_workspace_size", "ham_rnn_backward")
HAM_PROFILE_STAGES = 5


class HamDims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int),
                ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("io_dtype", ctypes.c_int),
                ("scale", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("cap", ctypes.c_int), ("flags", ctypes.c_int), ("t0", ctypes.c_int),
                ("rope_base", ctypes.c_float), ("route_block", ctypes.c_int),
                ("kv_heads", ctypes.c_int), ("dk_kv", ctypes.c_int), ("dv_kv", ctypes.c_int)]


class HamError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"HAM error {code}: {msg}")
        self.code = code


_lib = None


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python attention_sequence_mixing_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    D = ctypes.POINTER(HamDims)
    L.ham_version.restype = I
    L.ham_version.argtypes = []
    L.ham_last_error.restype = ctypes.c_char_p
    L.ham_last_error.argtypes = []
    for name in ("ham_forward_workspace_size", "ham_decode_workspace_size",
                 "ham_route_stats_workspace_size", "ham_attention_backward_workspace_size",
                 "ham_rnn_backward_workspace_size"):
        f = getattr(L, name)
        f.restype = Z
        f.argtypes = [D]
    L.ham_forward.restype = I
    L.ham_forward.argtypes = [D] + [P] * 24 + [Z, P]
    L.ham_decode_step.restype = I
    L.ham_decode_step.argtypes = [D] + [P] * 26 + [Z, P]
    L.ham_decode_step_noalloc.restype = I
    L.ham_decode_step_noalloc.argtypes = [D] + [P] * 25 + [P]
    L.ham_decode_noalloc_scratch_bytes.restype = Z
    L.ham_decode_noalloc_scratch_bytes.argtypes = []
    L.ham_route_stats.restype = I
    L.ham_route_stats.argtypes = [D] + [P] * 11 + [ctypes.c_float, P, P, Z, P]
    L.ham_attention_backward.restype = I
    L.ham_attention_backward.argtypes = [D] + [P] * 10 + [P, Z, P]
    L.ham_rnn_backward.restype = I
    L.ham_rnn_backward.argtypes = [D] + [P] * 15 + [Z, P]
    L.ham_select_tau.restype = I
    L.ham_select_tau.argtypes = [D, P, ctypes.c_double, P, P]
    L.ham_profile_start.restype = I
    L.ham_profile_start.argtypes = [I]
    L.ham_profile_stop.restype = I
    L.ham_profile_stop.argtypes = [P, I, P, P]
    _lib = L
    return L


def check(rc):
    if rc != HAM_OK:
        msg = lib().ham_last_error().decode(errors="replace")
        raise HamError(rc, msg)
    return rc

"""ctypes loader of libattn.so.  Loading needs no GPU; the library links the
HIP runtime only.  There is no fallback: when the library is missing every
entry point raises."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_OK, ATTN_ERR_INVALID_ARG, ATTN_ERR_UNSUPPORTED, ATTN_ERR_HIP = 0, 1, 2, 3
ATTN_F32, ATTN_BF16 = 0, 1
ATTN_ACCUMULATE, ATTN_OUT_F32, ATTN_NO_TILE_SKIP = 1, 2, 4

# Every symbol include/attn.h declares.
EXPORTS = ("attn_fwd", "attn_fwd_ex", "attn_merge", "rope_apply", "attn_cast", "attn_ring_plan", "attn_ring_fwd",
           "attn_ring_fwd_ex", "attn_bwd", "attn_bwd_ex", "attn_ring_bwd", "attn_ring_bwd_ex", "attn_kv_append", "attn_decode",
           "attn_decode_noalloc", "attn_profile_start", "attn_profile_stop", "attn_release_scratch",
           "attn_last_error", "attn_version")


class RingCall(ctypes.Structure):
    _fields_ = [
        ("step", ctypes.c_int),
        ("block", ctypes.c_int),
        ("q_row0", ctypes.c_int),
        ("q_rows", ctypes.c_int),
        ("q_pos0", ctypes.c_longlong),
        ("kv_pos0", ctypes.c_longlong),
        ("kv_rows", ctypes.c_int),
        ("accumulate", ctypes.c_int),
    ]


class Variant(ctypes.Structure):
    """attn_variant: sliding window (-1 = no limit) and ALiBi slopes."""
    _fields_ = [
        ("window_left", ctypes.c_longlong),
        ("window_right", ctypes.c_longlong),
        ("alibi_slopes", ctypes.c_void_p),
    ]


class AttnError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"attn error {code}: {msg}")
        self.code = code


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, ll, u, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_uint, ctypes.c_double
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, i, vp, vp, d, i, u, vp]
    var = ctypes.POINTER(Variant)
    lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, i, vp, vp, d, i, u, var, vp]
    lib.attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, i, vp, vp, d, i, u, var, vp]
    lib.attn_ring_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, d, i, u, var, vp]
    lib.attn_ring_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, d, i, u, var, vp]
    lib.attn_kv_append.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, d, i, vp]
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, d, i, u, var, vp]
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, d, i, u, var, vp]
    lib.attn_merge.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp]
    lib.rope_apply.argtypes = [vp, vp, d, i, i, i, i, i, vp]
    lib.attn_cast.argtypes = [vp, vp, ll, i, vp]
    lib.attn_ring_plan.argtypes = [i, i, i, i, i, ctypes.POINTER(RingCall), i]
    lib.attn_ring_fwd.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, d, i, u, vp]
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, ll, ll, i, vp, vp, d, i, u, vp]
    lib.attn_ring_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, d, i, u, vp]
    lib.attn_profile_start.argtypes = [i]
    lib.attn_profile_stop.argtypes = [ctypes.POINTER(ctypes.c_float), i]
    lib.attn_release_scratch.argtypes = []
    for name in ("attn_fwd", "attn_fwd_ex", "attn_merge", "rope_apply", "attn_cast", "attn_ring_plan",
                 "attn_ring_fwd", "attn_ring_fwd_ex", "attn_bwd", "attn_bwd_ex", "attn_ring_bwd", "attn_ring_bwd_ex",
                 "attn_kv_append", "attn_decode", "attn_decode_noalloc",
                 "attn_profile_start", "attn_profile_stop", "attn_release_scratch", "attn_version"):
        getattr(lib, name).restype = ctypes.c_int
    lib.attn_last_error.argtypes = []
    lib.attn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def check(rc: int) -> None:
    if rc != ATTN_OK:
        raise AttnError(rc, load().attn_last_error().decode())

"""ctypes view of the C ABI in include/dr.h (loading, descriptor struct, status codes).

Only argument marshalling lives here: every step of the recurrence runs in libdr's HIP
kernels.  If the library is missing this module raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdr.so")

DR_OK = 0
DR_E_NULL = -1
DR_E_SHAPE = -2
DR_E_DTYPE = -3
DR_E_ALIGN = -4
DR_E_ALIAS = -5
DR_E_UNSUPPORTED = -6
DR_E_WORKSPACE = -7
DR_E_HIP = -8
DR_E_SCRATCH = -9

DR_F32 = 0
DR_BF16 = 1
DR_GATE_HEAD = 0
DR_GATE_CHANNEL = 1
DR_GATE_RATE_SQRT = 2

EXPORTS = (
    "dr_abi_version",
    "dr_status_str",
    "dr_chunk_fwd_workspace_bytes",
    "dr_chunk_fwd",
    "dr_chunk_fwd_noalloc_max_bytes",
    "dr_chunk_fwd_noalloc",
    "dr_chunk_fwd_varlen_workspace_bytes",
    "dr_chunk_fwd_varlen",
    "dr_chunk_bwd_workspace_bytes",
    "dr_chunk_bwd",
    "dr_chunk_bwd_varlen_workspace_bytes",
    "dr_chunk_bwd_varlen",
    "dr_decode_step",
)


class DrDesc(ctypes.Structure):
    _fields_ = [
        (name, ctypes.c_int32)
        for name in (
            "B", "T", "H", "dk", "dv", "chunk", "qkv_dtype", "o_dtype",
            "decay_kind", "erase_kind", "write_kind", "write_is_erase",
        )
    ]


class DrError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdr.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m gated_delta_rule_dr_amd.build`"
        )
    L = ctypes.CDLL(LIB_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.dr_abi_version.restype = ctypes.c_int
    L.dr_abi_version.argtypes = []
    L.dr_status_str.restype = ctypes.c_char_p
    L.dr_status_str.argtypes = [ctypes.c_int]
    L.dr_chunk_fwd_workspace_bytes.restype = sz
    L.dr_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(DrDesc)]
    L.dr_chunk_fwd.restype = ctypes.c_int
    L.dr_chunk_fwd.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 10 + [sz, vp]
    L.dr_chunk_fwd_noalloc_max_bytes.restype = sz
    L.dr_chunk_fwd_noalloc_max_bytes.argtypes = []
    L.dr_chunk_fwd_noalloc.restype = ctypes.c_int
    L.dr_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 10
    L.dr_chunk_fwd_varlen_workspace_bytes.restype = sz
    L.dr_chunk_fwd_varlen_workspace_bytes.argtypes = [ctypes.POINTER(DrDesc), ctypes.c_int32]
    L.dr_chunk_fwd_varlen.restype = ctypes.c_int
    L.dr_chunk_fwd_varlen.argtypes = [ctypes.POINTER(DrDesc), vp, ctypes.c_int32] + [vp] * 10 + [sz, vp]
    L.dr_chunk_bwd_workspace_bytes.restype = sz
    L.dr_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(DrDesc)]
    L.dr_chunk_bwd.restype = ctypes.c_int
    L.dr_chunk_bwd.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 17 + [sz, vp]
    L.dr_chunk_bwd_varlen_workspace_bytes.restype = sz
    L.dr_chunk_bwd_varlen_workspace_bytes.argtypes = [ctypes.POINTER(DrDesc), ctypes.c_int32]
    L.dr_chunk_bwd_varlen.restype = ctypes.c_int
    L.dr_chunk_bwd_varlen.argtypes = [ctypes.POINTER(DrDesc), vp, ctypes.c_int32] + [vp] * 17 + [sz, vp]
    L.dr_decode_step.restype = ctypes.c_int
    L.dr_decode_step.argtypes = [ctypes.POINTER(DrDesc)] + [vp] * 9
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().dr_status_str(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != DR_OK:
        raise DrError(fn, status, status_str(status))

"""ctypes binding of libhils.so (the C ABI in include/hils.h).

Argument marshalling only.  Loading fails loudly when the library is missing:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhils.so")

HILS_OK, HILS_E_ARG, HILS_E_UNSUPPORTED, HILS_E_WORKSPACE, HILS_E_HIP = range(5)
HILS_BF16, HILS_F32 = 0, 1
MODES = {"surrogate": 0, "landmark_key": 1, "exact": 2, "mean_pool": 3}
HILS_FLAG_GENERIC = 1
HILS_FLAG_UNION = 2
HILS_MAX_DECODE_QUERIES = 16

EXPORTED = ("hils_workspace_bytes", "hils_summarize", "hils_prefill", "hils_decode",
            "hils_summarize_paged", "hils_decode_paged", "hils_decode_multi_workspace_bytes",
            "hils_decode_multi", "hils_prefill_backward_workspace_bytes", "hils_prefill_backward",
            "hils_strerror", "hils_abi_version", "hils_profile_enable", "hils_profile_read",
            "hils_decode_noalloc")
HILS_NOALLOC_SCRATCH_BYTES = 64 << 20


class HilsCfg(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("N", ctypes.c_int32), ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32), ("S", ctypes.c_int32),
        ("W", ctypes.c_int32), ("K", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("mode", ctypes.c_int32), ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
    ]


class HilsError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m chunk_wise_hierarchical_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
        cfgp = ctypes.POINTER(HilsCfg)
        L.hils_workspace_bytes.argtypes = [cfgp, ctypes.c_int]
        L.hils_workspace_bytes.restype = sz
        L.hils_summarize.argtypes = [cfgp, vp, vp, i32, i32, vp, vp, vp]
        L.hils_summarize.restype = ctypes.c_int
        L.hils_prefill.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hils_prefill.restype = ctypes.c_int
        L.hils_decode.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hils_decode.restype = ctypes.c_int
        L.hils_decode_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.hils_decode_noalloc.restype = ctypes.c_int
        L.hils_summarize_paged.argtypes = [cfgp, vp, vp, vp, i32, i32, vp, vp, vp]
        L.hils_summarize_paged.restype = ctypes.c_int
        L.hils_decode_paged.argtypes = [cfgp, vp, vp, vp, vp, i32, vp, i32, vp, vp, vp, vp, vp, vp,
                                        sz, vp]
        L.hils_decode_paged.restype = ctypes.c_int
        L.hils_decode_multi_workspace_bytes.argtypes = [cfgp, i32]
        L.hils_decode_multi_workspace_bytes.restype = sz
        L.hils_decode_multi.argtypes = [cfgp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.hils_decode_multi.restype = ctypes.c_int
        L.hils_prefill_backward_workspace_bytes.argtypes = [cfgp]
        L.hils_prefill_backward_workspace_bytes.restype = sz
        L.hils_prefill_backward.argtypes = [cfgp] + [vp] * 14 + [vp, sz, vp]
        L.hils_prefill_backward.restype = ctypes.c_int
        L.hils_strerror.argtypes = [ctypes.c_int]
        L.hils_strerror.restype = ctypes.c_char_p
        L.hils_abi_version.argtypes = []
        L.hils_abi_version.restype = ctypes.c_int
        L.hils_profile_enable.argtypes = [ctypes.c_int]
        L.hils_profile_enable.restype = None
        L.hils_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.hils_profile_read.restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().hils_strerror(status).decode()


def profile_enable(on: bool) -> None:
    lib().hils_profile_enable(1 if on else 0)


def profile_read(cap: int = 4096):
    """[(kernel name, ms)] of the kernels enqueued since the last read (streams synchronised)."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    n = lib().hils_profile_read(names, ms, cap)
    return [(names[i].decode(), float(ms[i])) for i in range(min(n, cap))]


def check(status: int, what: str) -> None:
    if status != HILS_OK:
        raise HilsError(status, what)

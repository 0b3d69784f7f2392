"""ctypes binding of libxs_attn.so (include/xs_attn.h): argument marshalling only."""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libxs_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "xs_attn.h")
HEADER_PATHS = [HEADER_PATH, os.path.join(os.path.dirname(_PKG), "include", "xs_burst_gap.h"),
                os.path.join(os.path.dirname(_PKG), "include", "xs_ceiling.h")]

_lib = None


class XsAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"xs_attn status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load the built library; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with `python -m sequence_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        L.xs_attn_fwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
        L.xs_attn_fwd.restype = ci
        L.xs_attn_fwd_fp8.argtypes = [vp, vp, vp, cf, cf, cf, vp, ci, ci, ci, ci, ci, cf, vp]
        L.xs_attn_fwd_fp8.restype = ci
        sz = ctypes.c_size_t
        L.xs_attn_fwd_ws.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp, sz, vp]
        L.xs_attn_fwd_ws.restype = ci
        L.xs_attn_fwd_fp8_ws.argtypes = [vp, vp, vp, cf, cf, cf, vp, ci, ci, ci, ci, ci, cf, vp, sz, vp]
        L.xs_attn_fwd_fp8_ws.restype = ci
        L.xs_attn_fwd_ex.argtypes = [vp, vp, vp, ci, vp, vp, ci, ci, ci, ci, ci, cf, vp, sz, vp]
        L.xs_attn_fwd_ex.restype = ci
        L.xs_attn_fwd_fp8_ex.argtypes = [vp, vp, vp, ci, cf, cf, cf, vp, vp, ci, ci, ci, ci, ci, cf,
                                         vp, sz, vp]
        L.xs_attn_fwd_fp8_ex.restype = ci
        L.xs_attn_fwd_noalloc.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
        L.xs_attn_fwd_noalloc.restype = ci
        L.xs_attn_workspace_size.argtypes = [ci, ci, ci, ci]
        L.xs_attn_workspace_size.restype = sz
        ip = ctypes.POINTER(ci)
        L.xs_attn_schedule.argtypes = [ci, ci, ci, ci, ci, ip, ip, ip]
        L.xs_attn_schedule.restype = ci
        L.xs_attn_schedule_ex.argtypes = [ci, ci, ci, ci, ci, ci, ip, ip, ip, ip]
        L.xs_attn_schedule_ex.restype = ci
        L.xs_attn_split_count.argtypes = [ci, ci, ci, ci]
        L.xs_attn_split_count.restype = ci
        L.xs_attn_strerror.argtypes = [ci]
        L.xs_attn_strerror.restype = ctypes.c_char_p
        L.xs_attn_version.argtypes = []
        L.xs_attn_version.restype = ci
        L.xs_burst_gap.argtypes = [vp, sz, ci, sz, ci, ctypes.c_longlong, vp, vp]
        L.xs_burst_gap.restype = ci
        L.xs_burst_gap_tiles.argtypes = [vp, sz, ci, ci, ci, ci, ctypes.c_longlong, ci, vp, sz, ci,
                                         vp, vp]
        L.xs_burst_gap_tiles.restype = ci
        L.xs_mfma_ceiling.argtypes = [ci, ci, ci, vp, sz, vp]
        L.xs_mfma_ceiling.restype = ci
        L.xs_clock_sample.argtypes = [vp, sz, ip, vp]
        L.xs_clock_sample.restype = ci
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().xs_attn_strerror(int(status)).decode()


def check(status: int) -> None:
    if status != 0:
        raise XsAttnError(status, strerror(status))


def declared_functions() -> list[str]:
    """Names of the functions declared in include/*.h."""
    names = []
    for path in HEADER_PATHS:
        text = open(path).read()
        names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(xs_\w+)\s*\(", text, flags=re.M)
    return names

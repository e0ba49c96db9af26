"""ctypes loader for the cpattn C-ABI library (libcpattn.so, built in-tree).

There is no fallback: if the library is missing every call raises.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
LIB_NAME = "libcpattn.so"
HEADER = os.path.join(_ROOT, "include", "cpattn.h")

BF16 = 0
FP32 = 1
FP16 = 2

STATUS = {
    0: "CPATTN_OK", 1: "CPATTN_ERR_NULL", 2: "CPATTN_ERR_SHAPE", 3: "CPATTN_ERR_DEGREE",
    4: "CPATTN_ERR_INDIVISIBLE", 5: "CPATTN_ERR_CHUNKS", 6: "CPATTN_ERR_DTYPE",
    7: "CPATTN_ERR_WORKSPACE", 8: "CPATTN_ERR_ALIAS", 9: "CPATTN_ERR_HIP",
}

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_fp = ctypes.POINTER(ctypes.c_float)

_SIGNATURES = {
    "cpattn_block_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp]),
    "cpattn_lse_merge": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, ctypes.c_int, _vp]),
    "cpattn_ring_fwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int]),
    "cpattn_ring_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float,
                                        ctypes.c_int, ctypes.POINTER(_i64), _vp, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_int, _vp]),
    "cpattn_ring_fwd_cfg": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, ctypes.c_float,
                                            ctypes.c_int, ctypes.POINTER(_i64), ctypes.c_int, _vp, ctypes.c_size_t,
                                            ctypes.c_int, ctypes.c_int, _vp]),
    "cpattn_ring_fwd_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64,
                                                ctypes.c_float, ctypes.c_int, ctypes.POINTER(_i64), ctypes.c_int,
                                                ctypes.c_int, _vp]),
    "cpattn_ring_fwd_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "cpattn_ulysses_permute": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, _i64, _vp]),
    "cpattn_ulysses_anything_permute": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, ctypes.c_int,
                                                        ctypes.POINTER(_i64), ctypes.POINTER(_i64), ctypes.c_int,
                                                        ctypes.c_int, _i64, _vp]),
    "cpattn_unified_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _vp,
                                           ctypes.c_size_t, ctypes.c_int, ctypes.c_int, _vp]),
    "cpattn_unified_fwd_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _i64, _i64, ctypes.c_int, ctypes.c_int,
                                                              ctypes.c_int, ctypes.c_int]),
    "cpattn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "cpattn_last_error": (ctypes.c_char_p, []),
    "cpattn_version": (ctypes.c_int, []),
}

_lib = None


def library_path() -> str:
    return os.path.join(_HERE, LIB_NAME)


def declared_functions(header: str = HEADER):
    """Names of the functions include/cpattn.h declares."""
    with open(header) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpattn_[a-z0-9_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"cpattn HIP library is not built ({path} is missing); "
                               "run __graft_entry__.build() first")
        L = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class CpattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS.get(status, str(status))


def check(status: int) -> None:
    if status != 0:
        msg = lib().cpattn_last_error().decode(errors="replace")
        raise CpattnError(status, msg)

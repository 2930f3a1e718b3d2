"""ctypes loader for the HIP library (libspecverify.so, built for gfx950 next to this file).

There is no fallback: if the library is missing or fails to load, importing the binding
raises, so nothing can silently run another implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_NAME = "libspecverify.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

SV_OK, SV_EINVAL, SV_EDTYPE, SV_EHIP, SV_ENODEV, SV_ENOMEM, SV_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
SV_NOALLOC_SCRATCH_BYTES = 32 << 20
SV_MAX_D = 31
DTYPE_F32, DTYPE_BF16 = 0, 1

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

# every exported symbol with its argument and result types
SIGNATURES = {
    "spec_verify_bf16": ([_p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p], _i),
    "spec_verify_f32": ([_p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p], _i),
    "spec_verify_workspace_bytes": ([_i, _i, _i], _sz),
    "spec_verify_ws": ([_i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _sz, _p], _i),
    "spec_verify_noalloc": ([_i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p], _i),
    "spec_verify_debug": ([_i, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p], _i),
    "spec_verify_advance": ([_p, _p, _i, _i, _p, _i, _p, _p], _i),
    "spec_verify_threshold": ([_i, _p, _p, _p, _p, _i, _i, _i, _p, ctypes.c_float, _p, _p, _p],
                              _i),
    "spec_verify_saguaro_reshape": ([_i, _p, _p, _p, _i, _i, _i, ctypes.c_float, _i, _p], _i),
    "spec_verify_saguaro_workspace_bytes": ([_i, _i, _i], _sz),
    "spec_verify_saguaro_reshape_ws": ([_i, _p, _p, _p, _i, _i, _i, ctypes.c_float, _i, _p, _sz,
                                        _p], _i),
    "spec_verify_strerror": ([_i], ctypes.c_char_p),
    "spec_verify_version": ([], _i),
    "spec_verify_release": ([_p], _i),
    "spec_verify_row_stages": ([_i, _i, _i, _i, _p, _i], _i),
    "spec_verify_profile_start": ([_i], _i),
    "spec_verify_profile_stop": ([_p, _i, _p], _i),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load (once) and return the library. Raises ImportError if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it first (__graft_entry__.build())")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = res
        _lib = handle
    return _lib


def strerror(code: int) -> str:
    return lib().spec_verify_strerror(code).decode()


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {strerror(code)} ({code})")
        self.code = code

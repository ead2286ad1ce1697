"""ctypes view of liblwg.so (the C ABI declared in include/lwg.h).

The library is looked up next to this file (built in place by
``python -m layernorm_window_gather_amd.build``) or at ``$LWG_LIBRARY``. A
missing library is an error: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("LWG_LIBRARY", os.path.join(_HERE, "liblwg.so"))

# status codes of lwg_status
LWG_OK = 0
LWG_ERR_INVALID_ARGUMENT = 1
LWG_ERR_UNSUPPORTED_WIDTH = 2
LWG_ERR_MISALIGNED = 3
LWG_ERR_ALIASING = 4
LWG_ERR_SIZE_MISMATCH = 5
LWG_ERR_HIP = 6

_i32, _i64, _f64, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p

# name -> (restype, argtypes); must list every function of include/lwg.h
SIGNATURES = {
    "lwg_ln_fixed": (_i32, [_p, _p, _i64, _i32, _f64, _p]),
    "lwg_add_ln": (_i32, [_p, _p, _p, _p, _i64, _i32, _f64, _p]),
    "lwg_window_token_count": (_i64, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "lwg_window_index_build": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _p, _i64, _p]),
    "lwg_window_gather": (_i32, [_p, _i64, _i32, _p, _i64, _p, _p]),
    "lwg_norm_gather": (_i32, [_p, _i64, _i32, _p, _i64, _f64, _p, _p]),
    "lwg_window_inverse_build": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                        _p, _i64, _p]),
    "lwg_window_reverse_add_ln": (_i32, [_p, _i64, _p, _p, _p, _p, _i64, _i32, _f64, _p]),
    "lwg_add_norm_gather": (_i32, [_p, _p, _p, _i64, _i32, _p, _i64, _f64, _p, _p]),
    "lwg_ln_affine": (_i32, [_p, _p, _p, _p, _i64, _i32, _f64, _p]),
    "lwg_bias_gelu": (_i32, [_p, _p, _p, _i64, _i32, _p]),
    "lwg_add_ln_affine": (_i32, [_p, _p, _p, _p, _p, _p, _i64, _i32, _f64, _p]),
    "lwg_status_string": (ctypes.c_char_p, [_i32]),
    "lwg_last_error": (ctypes.c_char_p, []),
    "lwg_abi_version": (_i32, []),
}

ABI_VERSION = 1

_lock = threading.Lock()
_handle = None


class LwgError(RuntimeError):
    """A non-OK status from the library; ``status`` holds the lwg_status code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load():
    """Load liblwg.so once and attach the signatures. Raises if it is absent."""
    global _handle
    with _lock:
        if _handle is not None:
            return _handle
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"liblwg.so not found at {LIB_PATH}; build it with "
                "`python -m layernorm_window_gather_amd.build` (there is no fallback path)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.lwg_abi_version() != ABI_VERSION:
            raise RuntimeError(f"liblwg.so ABI version {lib.lwg_abi_version()} != {ABI_VERSION}")
        _handle = lib
        return lib


def check(status: int) -> None:
    """Raise LwgError for a non-OK status, with the library's own message."""
    if status != LWG_OK:
        lib = load()
        name = lib.lwg_status_string(status).decode()
        detail = lib.lwg_last_error().decode()
        raise LwgError(status, f"{name}: {detail}")

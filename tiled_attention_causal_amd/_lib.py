"""ctypes loader for libfa.so (the C ABI declared in include/fa.h).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
There is no fallback; if the library is missing the import of any entry point fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import threading

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_SUCCESS = 0
FA_ERROR_INVALID_VALUE = 1
FA_ERROR_NOT_SUPPORTED = 2
FA_ERROR_LAUNCH_FAILED = 3
FA_ERROR_SCRATCH_TOO_SMALL = 4
FA_BACKWARD_NOALLOC_MAX_BYTES = 32 << 20

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1

# Every symbol include/fa.h declares, with its ctypes signature.
_i64 = ctypes.c_int64
_ptr = ctypes.c_void_p
SIGNATURES = {
    "fa_forward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                     ctypes.c_int]),
    "fa_forward": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr,
                                  ctypes.c_int, ctypes.c_float, _ptr, _ptr, _ptr]),
    "fa_forward_with_workspace": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                 _ptr, _ptr, _ptr, ctypes.c_int, ctypes.c_float,
                                                 _ptr, _ptr, _ptr, ctypes.c_size_t, _ptr]),
    "fa_backward_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64]),
    "fa_backward": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr,
                                   _ptr, _ptr, _ptr, ctypes.c_int, ctypes.c_float, _ptr, _ptr,
                                   _ptr, _ptr, ctypes.c_size_t, _ptr]),
    "fa_backward_atomic_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int, _i64, _i64, _i64, _i64,
                                                             _i64]),
    "fa_backward_atomic": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr, _ptr,
                                          _ptr, _ptr, _ptr, _ptr, ctypes.c_int, ctypes.c_float,
                                          _ptr, _ptr, _ptr, _ptr, ctypes.c_size_t, _ptr]),
    "fa_backward_preprocess": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _ptr, _ptr,
                                              _ptr, _ptr, ctypes.c_size_t, _ptr]),
    "fa_backward_main": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr, _ptr,
                                        _ptr, _ptr, _ptr, _ptr, ctypes.c_int, ctypes.c_float,
                                        _ptr, _ptr, _ptr, _ptr, ctypes.c_size_t, _ptr]),
    "fa_backward_noalloc": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _ptr,
                                           _ptr, _ptr, _ptr, _ptr, _ptr, ctypes.c_int,
                                           ctypes.c_float, _ptr, _ptr, _ptr, _ptr]),
    "fa_forward_kernel_name": (ctypes.c_char_p, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                 ctypes.c_int, ctypes.c_size_t]),
    "fa_backward_kernel_name": (ctypes.c_char_p, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                  ctypes.c_int, ctypes.c_size_t]),
    "fa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
}

_lock = threading.Lock()
_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where} failed: {status_string(status)} ({status})")


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m "
                    "tiled_attention_causal_amd.build` (hipcc, gfx950). There is no fallback.")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().fa_status_string(status).decode()

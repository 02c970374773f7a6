"""ctypes loader for libpagedattn.so (the C ABI in include/pagedattn.h).

Loading needs only the HIP runtime library, not a GPU. The library is never
rebuilt here: a missing library raises, it is not replaced by anything else.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")
# Read-bandwidth calibration kernels (include/pa_calib.h), used by the benchmark only.
CALIB_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpacalib.so")

_i32 = ctypes.c_int32
_ptr = ctypes.c_void_p
_f32 = ctypes.c_float
_size = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/pagedattn.h
SIGNATURES = {
    "pa_reshape_and_cache": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _ptr]),
    "pa_decode_workspace_size": (_size, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _f32, _i32, _i32, _i32, _i32, _i32,
                         _i32, _i32, _i32, _i32, _i32, _ptr, _size, _ptr]),
    "pa_decode_step": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _f32, _i32,
                              _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ptr, _size,
                              _ptr]),
    "pa_decode_step_noalloc": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _f32,
                                      _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _ptr]),
    "pa_copy_blocks": (_i32, [_ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32, _i32, _ptr]),
    "pa_swap_blocks": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _i32, _i32, _i32, _i32, _i32,
                              _i32, _i32, _ptr]),
    "pa_prefill": (_i32, [_ptr, _ptr, _ptr, _ptr, _ptr, _ptr, _ptr, ctypes.c_float, _i32, _i32,
                          _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _ptr]),
    "pa_status_str": (ctypes.c_char_p, [_i32]),
    "pa_abi_version": (_i32, []),
}

CALIB_SIGNATURES = {
    "pa_calib_stream_read": (_i32, [_ptr, _size, _i32, _i32, _ptr, _ptr]),
    "pa_calib_tile_read": (_i32, [_ptr, ctypes.c_int64, _ptr, _i32, _i32, _i32, _i32, _ptr, _ptr]),
}

_LIB = None
_CALIB = None


class LibraryNotBuilt(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise LibraryNotBuilt(
                f"{LIB_PATH} is missing; build it with `python -m paged_kv_cache_362_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def calib_lib() -> ctypes.CDLL:
    global _CALIB
    if _CALIB is None:
        if not os.path.exists(CALIB_LIB_PATH):
            raise LibraryNotBuilt(
                f"{CALIB_LIB_PATH} is missing; build it with "
                f"`python -m paged_kv_cache_362_amd.build`")
        handle = ctypes.CDLL(CALIB_LIB_PATH)
        for name, (res, args) in CALIB_SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _CALIB = handle
    return _CALIB


def status_str(code: int) -> str:
    return lib().pa_status_str(code).decode()

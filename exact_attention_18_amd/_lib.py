"""ctypes loader for libfa.so: the C ABI declared in include/fa.h.

Loading the library needs no GPU.  If the library has not been built the
loader raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = -1
FA_ERR_UNSUPPORTED = -2
FA_ERR_HIP = -3
FA_ERR_TOO_LARGE = -4
NOALLOC_SCRATCH_BYTES = 16 << 20

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/fa.h
SIGNATURES = {
    "fa_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_forward_block_sparse": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_block_sparse_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_decode_workspace_size": (_sz, [_i, _i, _i, _i, _i]),
    "fa_fp8_buffer_size": (_sz, [_i, _i, _i, _i]),
    "fa_fp8_prepare": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "fa_forward_fp8_prepared": (_i, [_vp, _sz, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "fa_forward_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                         _vp, _sz, _vp]),
    "fa_backward_preprocess": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _sz, _vp]),
    "fa_backward_dkdv": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_backward_dq": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_backward_dq_delta": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp]),
    "fa_backward_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_backward_atomic_workspace_size": (_sz, [_i, _i, _i, _i]),
    "fa_backward_atomic": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                                _vp, _sz, _vp]),
    "fa_backward_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_forward_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp]),
    "fa_backward_f32": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f,
                             _vp, _sz, _vp]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
    "fa_abi_version": (_i, []),
}

_lib = None


class FaLibraryMissing(RuntimeError):
    pass


def load() -> ctypes.CDLL:
    """Load libfa.so once and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FaLibraryMissing(
            f"{LIB_PATH} is not built; run `python -m exact_attention_18_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib

"""ctypes loader for libfa.so (the C ABI declared in include/fa.h).

The library is built in-tree (exact_io_aware_08_amd/libfa.so).  If it is not
there, loading builds it with hipcc; if that fails the import raises -- there
is no other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_HEADDIM", 4: "FA_ERR_GQA",
    5: "FA_ERR_DTYPE", 6: "FA_ERR_ALIGN", 7: "FA_ERR_SCALE", 8: "FA_ERR_WORKSPACE",
    9: "FA_ERR_DEVICE", 10: "FA_ERR_HIP", 11: "FA_ERR_ARG", 12: "FA_ERR_SCRATCH",
}

_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_sz = ctypes.c_size_t

# name -> (restype, argtypes); mirrors include/fa.h
SIGNATURES = {
    "fa_fwd": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp]),
    "fa_fwd_pcast": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _f, _i,
                          _i, _vp, _vp]),
    "fa_kv_tile": (_i, [_i, _i, _i]),
    "fa_decode_splits": (_i, [_i, _i, _i, _i, _i]),
    "fa_decode_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "fa_decode_paged_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i, _i]),
    "fa_decode": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp, _sz, _vp]),
    "fa_decode_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp]),
    "fa_cast_e4m3": (_i, [_vp, _vp, _vp, _sz, _vp]),
    "fa_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "fa_decode_paged": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                             _i, _i, _vp, _sz, _vp]),
    "fa_bwd": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f,
                    _i, _vp, _sz, _vp]),
    "fa_quant_e4m3": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "fa_fp8_kv_tile": (_i, []),
    "fa_fwd_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _f,
                        _i, _i, _vp]),
    "fa_status_str": (ctypes.c_char_p, [_i]),
    "fa_version": (_i, []),
}

_lib = None


def load(path: str | None = None):
    """Load libfa.so (building it first if it is missing)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = load().fa_status_str(status).decode()
        super().__init__(f"{where}: {msg}")


def check(status: int, where: str) -> None:
    if status != FA_OK:
        raise FaError(status, where)

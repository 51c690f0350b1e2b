"""ctypes loader for libfa.so (the C ABI declared in include/fa.h).

The library is built in-tree (``io_aware_tiled_05_amd/libfa.so``).  There is
no fallback: if it is missing, every call raises.
"""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK, FA_ERR_INVALID, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, -1, -2, -3, -4
FA_NOALLOC_SCRATCH_BYTES = 128 << 20
FA_BWD_STAGE_D, FA_BWD_STAGE_DKDV, FA_BWD_STAGE_DQ, FA_BWD_STAGE_GRADS = 1, 2, 3, 4



class FaStrides(C.Structure):
    """fa_strides: element strides (batch, head, row) of a [B][H][N][d] view."""
    _fields_ = [("batch", C.c_int64), ("head", C.c_int64), ("row", C.c_int64)]


class FaLayout(C.Structure):
    """fa_layout: the strides of every tensor of a call."""
    _fields_ = [(n, FaStrides) for n in ("q", "k", "v", "o", "dO", "dq", "dk", "dv")]


# (name, restype, argtypes) for every function in include/fa.h
_P, _I, _F, _SZ = C.c_void_p, C.c_int, C.c_float, C.c_size_t
_LP = C.POINTER(FaLayout)
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I, _P]),
    "fa_bwd_workspace_size": (_SZ, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P,
                    _SZ, _I, _P]),
    "fa_fwd_blocksparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P, _I, _I, _P]),
    "fa_bwd_blocksparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _P,
                                _I, _P, _SZ, _I, _P]),
    "fa_bwd_stage": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P,
                          _P, _I, _P, _SZ, _I, _P]),
    "fa_fwd_dropout": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _F, C.c_uint64,
                            C.c_uint32, _I, _P]),
    "fa_bwd_dropout": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _F,
                            C.c_uint64, C.c_uint32, _P, _SZ, _I, _P]),
    "fa_decode_workspace_size": (_SZ, [_I, _I, _I, _I, _I]),
    "fa_decode": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P, _SZ, _I, _P]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _I,
                            _P]),
    "fa_fwd_strided": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P, _I, _F,
                            C.c_uint64, C.c_uint32, _LP, _I, _P]),
    "fa_bwd_strided": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _F, _I, _P, _P,
                            _I, _F, C.c_uint64, C.c_uint32, _LP, _P, _SZ, _I, _P]),
    "fa_status_string": (C.c_char_p, [_I]),
}

_lib = None


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def load():
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m io_aware_tiled_05_amd.build` (hipcc, gfx950)")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(fn: str, status: int):
    if status != FA_OK:
        msg = load().fa_status_string(status).decode()
        raise FaError(fn, status, msg)

"""ctypes loader of libtq.so and the C-ABI signatures of include/tq.h.

This module only loads the library.  It raises if the HIP library is missing:
there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libtq.so")

TQ_OK, TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_ERR_DTYPE, TQ_ERR_ALIGN, TQ_ERR_LAUNCH, TQ_ERR_DEVICE, \
    TQ_ERR_FLAGS = range(8)
TQ_F32, TQ_BF16 = 0, 1
TQ_AMAX_GIVEN = 1

# name -> (restype, argtypes), matching include/tq.h
_P = C.c_void_p
_I64 = C.c_int64
_I32 = C.c_int32
_U32 = C.c_uint32
SIGNATURES = {
    "tq_tensor_amax": (_I32, [_P, _I32, _I64, _I64, _P, _P]),
    "tq_quantize": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _U32, _P]),
    "tq_extract_hint": (_I32, [_P, _I64, _P, _P]),
    "tq_quantize_guided": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P, _U32, _P]),
    "tq_requant_transpose_sr": (_I32, [_P, _P, _P, _I64, _I64, _I64, C.c_uint64, _P, _P, _P, _P]),
    "tq_grouped_gemm_nvfp4": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "tq_quantize_mxfp8": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P]),
    "tq_requant_transpose_mxfp8_sr": (_I32, [_P, _P, _P, _I64, _I64, _I64, C.c_uint64, _P, _P, _P, _P]),
    "tq_quantize_tile16": (_I32, [_P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _U32, _P]),
    "tq_transpose_tile16": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "tq_grouped_gemm_w4a4": (_I32, [_P, _P, _P, _P, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "tq_dequantize": (_I32, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "tq_code_mismatch": (_I32, [_P, _P, _I64, _I64, _P, _P]),
    "tq_hint_first_layer": (_I32, [_I32]),
    "tq_status_string": (C.c_char_p, [_I32]),
    "tq_version": (_I32, []),
}

_lib = None


class TqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {lib().tq_status_string(status).decode()}")


def lib():
    """The loaded libtq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libtq.so not found at {LIB_PATH}; build it with "
                "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int, where: str):
    if status != TQ_OK:
        raise TqError(status, where)

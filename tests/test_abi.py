"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/tq.h, and rejects bad arguments synchronously, before any
HIP call (every call below fails validation, so no pointer is dereferenced)."""
import ctypes as C
import os
import re

import pytest

from fp4_quantization_precision_amd import _lib
from fp4_quantization_precision_amd._lib import (TQ_BF16, TQ_ERR_ALIGN, TQ_ERR_DTYPE, TQ_ERR_FLAGS,
                                                 TQ_ERR_NULL, TQ_ERR_SHAPE, TQ_F32, TQ_OK)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq.h")

# fake device addresses: never dereferenced, only checked for null/alignment
P = C.c_void_p(0x7F0000000000)
P_MIS = C.c_void_p(0x7F0000000001)
NULL = None


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"TQ_API\s+[\w\s\*]+?\b(tq_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ["tq_quantize", "tq_extract_hint", "tq_quantize_guided",
                     "tq_requant_transpose_sr", "tq_grouped_gemm_nvfp4", "tq_grouped_gemm_w4a4"]:
        assert required in names
    assert set(names) == set(_lib.SIGNATURES), "binding signatures out of sync with tq.h"


def test_library_exports_every_declared_symbol(L):
    out = os.popen(f"nm -D --defined-only {_lib.LIB_PATH}").read()
    exported = set(re.findall(r"\bT (tq_\w+)", out))
    assert set(declared_functions()) <= exported
    # nothing but the C ABI is exported
    assert exported == set(declared_functions())


def test_host_only_helpers(L):
    assert L.tq_version() == 0x000100
    assert [L.tq_hint_first_layer(n) for n in (48, 47, 2, 1, 0, -3)] == [24, 23, 1, 0, 0, 0]
    for s in range(8):
        assert L.tq_status_string(s).startswith(b"TQ_")
    assert L.tq_status_string(99) == b"unknown tq_status"


def q(L, x=P, dtype=TQ_BF16, batch=1, rows=16, cols=32, amax=P, codes=P, scales=P, ts=P, hints=NULL,
      flags=0):
    return L.tq_quantize(x, dtype, batch, rows, cols, amax, codes, scales, ts, hints, flags, NULL)


def test_quantize_validation(L):
    assert q(L, dtype=7) == TQ_ERR_DTYPE
    assert q(L, flags=2) == TQ_ERR_FLAGS
    assert q(L, cols=24) == TQ_ERR_SHAPE
    assert q(L, rows=-1) == TQ_ERR_SHAPE
    assert q(L, batch=-2) == TQ_ERR_SHAPE
    assert q(L, batch=2 ** 40, rows=2 ** 20, cols=2 ** 20) == TQ_ERR_SHAPE  # overflow
    assert q(L, x=NULL) == TQ_ERR_NULL
    assert q(L, codes=NULL) == TQ_ERR_NULL
    assert q(L, scales=NULL) == TQ_ERR_NULL
    assert q(L, ts=NULL) == TQ_ERR_NULL
    assert q(L, amax=NULL) == TQ_ERR_NULL
    assert q(L, x=P_MIS) == TQ_ERR_ALIGN
    assert q(L, codes=P_MIS) == TQ_ERR_ALIGN
    assert q(L, hints=P_MIS) == TQ_ERR_ALIGN
    assert q(L, batch=0) == TQ_OK  # nothing to do, nothing launched
    assert q(L, dtype=TQ_F32, cols=16, x=NULL) == TQ_ERR_NULL


def test_guided_validation(L):
    g = L.tq_quantize_guided
    assert g(P, 5, 1, 16, 32, P, NULL, P, P, P, 0, NULL) == TQ_ERR_DTYPE
    assert g(P, TQ_BF16, 1, 16, 40, P, NULL, P, P, P, 0, NULL) == TQ_ERR_SHAPE
    assert g(P, TQ_BF16, 1, 16, 32, P, P_MIS, P, P, P, 0, NULL) == TQ_ERR_ALIGN
    assert g(NULL, TQ_BF16, 1, 16, 32, P, P, P, P, P, 0, NULL) == TQ_ERR_NULL
    assert g(P, TQ_BF16, 1, 16, 32, P, P, P, P, P, 4, NULL) == TQ_ERR_FLAGS


def test_extract_hint_validation(L):
    f = L.tq_extract_hint
    assert f(P, -1, P, NULL) == TQ_ERR_SHAPE
    assert f(NULL, 64, P, NULL) == TQ_ERR_NULL
    assert f(P, 64, NULL, NULL) == TQ_ERR_NULL
    assert f(P_MIS, 64, P, NULL) == TQ_ERR_ALIGN
    assert f(P, 64, C.c_void_p(0x7F0000000002), NULL) == TQ_ERR_ALIGN
    assert f(NULL, 0, NULL, NULL) == TQ_OK


def test_sr_validation(L):
    f = L.tq_requant_transpose_sr
    assert f(P, P, P, 1, 24, 32, 0, P, P, P, NULL) == TQ_ERR_SHAPE   # rows % 16
    assert f(P, P, P, 1, 32, 24, 0, P, P, P, NULL) == TQ_ERR_SHAPE   # cols % 16
    assert f(P, P, P, -1, 32, 32, 0, P, P, P, NULL) == TQ_ERR_SHAPE
    assert f(NULL, P, P, 1, 32, 32, 0, P, P, P, NULL) == TQ_ERR_NULL
    assert f(P, P, P, 1, 32, 32, 0, NULL, P, P, NULL) == TQ_ERR_NULL
    assert f(P, P, NULL, 1, 32, 32, 0, P, P, P, NULL) == TQ_ERR_NULL
    assert f(P_MIS, P, P, 1, 32, 32, 0, P, P, P, NULL) == TQ_ERR_ALIGN
    assert f(P, P, P, 1, 32, 32, 0, P_MIS, P, P, NULL) == TQ_ERR_ALIGN
    assert f(NULL, NULL, NULL, 0, 32, 32, 0, NULL, NULL, NULL, NULL) == TQ_OK


def test_gemm_validation(L):
    f = L.tq_grouped_gemm_nvfp4
    ok = dict(a=P, off=P, g=2, m=64, n=64, k=64, wc=P, ws=P, wt=P, out=P)

    def call(**kw):
        d = dict(ok, **kw)
        return f(d["a"], d["off"], d["g"], d["m"], d["n"], d["k"], d["wc"], d["ws"], d["wt"],
                 d["out"], NULL)

    assert call(g=0) == TQ_ERR_SHAPE
    assert call(k=40) == TQ_ERR_SHAPE
    assert call(k=(1 << 22) + 16) == TQ_ERR_SHAPE
    assert call(n=63) == TQ_ERR_SHAPE
    assert call(m=-1) == TQ_ERR_SHAPE
    assert call(m=2 ** 31) == TQ_ERR_SHAPE                      # beyond int32 group offsets
    assert call(m=2 ** 31 - 1, n=2 ** 26, k=16) == TQ_ERR_SHAPE  # tile count beyond 32 bits
    assert call(off=NULL) == TQ_ERR_NULL
    assert call(a=NULL) == TQ_ERR_NULL
    assert call(wc=NULL) == TQ_ERR_NULL
    assert call(out=NULL) == TQ_ERR_NULL
    assert call(wt=NULL) == TQ_ERR_NULL
    assert call(a=P_MIS) == TQ_ERR_ALIGN
    assert call(wc=P_MIS) == TQ_ERR_ALIGN
    assert call(out=C.c_void_p(0x7F0000000002)) == TQ_ERR_ALIGN
    assert call(m=0) == TQ_OK and call(n=0) == TQ_OK


def test_w4a4_gemm_validation(L):
    f = L.tq_grouped_gemm_w4a4
    ok = dict(ac=P, as_=P, at=P, off=P, g=2, m=64, n=64, k=64, wc=P, ws=P, wt=P, out=P)

    def call(**kw):
        d = dict(ok, **kw)
        return f(d["ac"], d["as_"], d["at"], d["off"], d["g"], d["m"], d["n"], d["k"], d["wc"],
                 d["ws"], d["wt"], d["out"], NULL)

    assert call(g=0) == TQ_ERR_SHAPE
    assert call(k=40) == TQ_ERR_SHAPE
    assert call(k=(1 << 22) + 16) == TQ_ERR_SHAPE
    assert call(n=63) == TQ_ERR_SHAPE
    assert call(m=2 ** 31) == TQ_ERR_SHAPE
    assert call(m=2 ** 31 - 1, n=2 ** 26, k=16) == TQ_ERR_SHAPE
    assert call(off=NULL) == TQ_ERR_NULL
    assert call(ac=NULL) == TQ_ERR_NULL
    assert call(as_=NULL) == TQ_ERR_NULL
    assert call(at=NULL) == TQ_ERR_NULL
    assert call(wc=NULL) == TQ_ERR_NULL
    assert call(out=NULL) == TQ_ERR_NULL
    assert call(ac=P_MIS) == TQ_ERR_ALIGN
    assert call(wc=P_MIS) == TQ_ERR_ALIGN
    assert call(m=0) == TQ_OK and call(n=0) == TQ_OK


def test_mxfp8_validation(L):
    q = L.tq_quantize_mxfp8
    assert q(P, 5, 1, 4, 64, P, P, NULL) == TQ_ERR_DTYPE
    assert q(P, TQ_BF16, 1, 4, 48, P, P, NULL) == TQ_ERR_SHAPE  # cols % 32
    assert q(NULL, TQ_BF16, 1, 4, 64, P, P, NULL) == TQ_ERR_NULL
    assert q(P, TQ_BF16, 1, 4, 64, P, NULL, NULL) == TQ_ERR_NULL
    assert q(P_MIS, TQ_BF16, 1, 4, 64, P, P, NULL) == TQ_ERR_ALIGN
    assert q(NULL, TQ_BF16, 0, 4, 64, NULL, NULL, NULL) == TQ_OK
    t = L.tq_requant_transpose_mxfp8_sr
    assert t(P, P, P, 1, 48, 32, 0, P, P, P, NULL) == TQ_ERR_SHAPE   # rows % 32
    assert t(P, P, P, 1, 64, 24, 0, P, P, P, NULL) == TQ_ERR_SHAPE   # cols % 16
    assert t(P, P, NULL, 1, 64, 32, 0, P, P, P, NULL) == TQ_ERR_NULL
    assert t(NULL, P, P, 1, 64, 32, 0, P, P, P, NULL) == TQ_ERR_NULL
    assert t(P_MIS, P, P, 1, 64, 32, 0, P, P, P, NULL) == TQ_ERR_ALIGN
    assert t(NULL, NULL, NULL, 0, 64, 32, 0, NULL, NULL, NULL, NULL) == TQ_OK


def test_tile16_validation(L):
    q = L.tq_quantize_tile16
    assert q(P, 7, 1, 16, 32, P, P, P, P, 0, NULL) == TQ_ERR_DTYPE
    assert q(P, TQ_BF16, 1, 24, 32, P, P, P, P, 0, NULL) == TQ_ERR_SHAPE   # rows % 16
    assert q(P, TQ_BF16, 1, 16, 40, P, P, P, P, 0, NULL) == TQ_ERR_SHAPE   # cols % 16
    assert q(P, TQ_BF16, 1, 16, 32, P, P, P, P, 2, NULL) == TQ_ERR_FLAGS
    assert q(NULL, TQ_BF16, 1, 16, 32, P, P, P, P, 0, NULL) == TQ_ERR_NULL
    assert q(P_MIS, TQ_BF16, 1, 16, 32, P, P, P, P, 0, NULL) == TQ_ERR_ALIGN
    assert q(P, TQ_BF16, 0, 16, 32, P, P, P, P, 0, NULL) == TQ_OK
    t = L.tq_transpose_tile16
    assert t(P, P, P, 1, 24, 32, P, P, P, NULL) == TQ_ERR_SHAPE
    assert t(NULL, P, P, 1, 16, 32, P, P, P, NULL) == TQ_ERR_NULL
    assert t(P, P, NULL, 1, 16, 32, P, P, P, NULL) == TQ_ERR_NULL
    assert t(C.c_void_p(0x7F0000000004), P, P, 1, 16, 32, P, P, P, NULL) == TQ_ERR_ALIGN
    assert t(NULL, NULL, NULL, 0, 16, 32, NULL, NULL, NULL, NULL) == TQ_OK


def test_other_validation(L):
    assert L.tq_tensor_amax(P, 9, 1, 32, P, NULL) == TQ_ERR_DTYPE
    assert L.tq_tensor_amax(P, TQ_BF16, 1, 24, P, NULL) == TQ_ERR_SHAPE
    assert L.tq_tensor_amax(P_MIS, TQ_BF16, 1, 32, P, NULL) == TQ_ERR_ALIGN
    assert L.tq_tensor_amax(P, TQ_BF16, 1, 32, NULL, NULL) == TQ_ERR_NULL
    assert L.tq_dequantize(P, P, P, 1, 16, 24, P, NULL) == TQ_ERR_SHAPE
    assert L.tq_dequantize(P, P, P, 1, 16, 32, P_MIS, NULL) == TQ_ERR_ALIGN
    assert L.tq_dequantize(P, NULL, P, 1, 16, 32, P, NULL) == TQ_ERR_NULL
    assert L.tq_code_mismatch(P, P, 1, 48, P, NULL) == TQ_ERR_SHAPE
    assert L.tq_code_mismatch(P, P_MIS, 1, 64, P, NULL) == TQ_ERR_ALIGN
    assert L.tq_code_mismatch(P, P, 1, 64, NULL, NULL) == TQ_ERR_NULL
    assert L.tq_code_mismatch(P, P, 1, 64, C.c_void_p(0x7F0000000004), NULL) == TQ_ERR_ALIGN


def test_binding_refuses_host_tensors():
    import torch
    from fp4_quantization_precision_amd import ops
    with pytest.raises(ValueError, match="device tensor"):
        ops.quantize(torch.zeros(16, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="device tensor"):
        ops.extract_hint(torch.zeros(16, dtype=torch.uint8), 32)

"""CPU oracle for the block-scaled FP4 path - TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  The product library never calls it; it shares no
source with the HIP kernels (``tq_oracle.c`` includes nothing from the
package).  This file only marshals numpy arrays into ``libtq_oracle.so``.

Every function returns numpy arrays.  Inputs may be numpy arrays or CPU torch
tensors; bf16 data is passed as its raw 16-bit patterns.

Parity status: every oracle function is pinned by tests against values fixed
independently of it (see tests/test_oracle_pins.py); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libtq_oracle.so")

F32, BF16 = 0, 1

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, IEEE binary32)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = C.CDLL(_LIB_PATH)
        p = C.c_void_p
        i64, i32 = C.c_int64, C.c_int
        L.tqo_e2m1_value.argtypes = [i32]
        L.tqo_e2m1_value.restype = C.c_double
        L.tqo_e4m3_value.argtypes = [C.c_uint8]
        L.tqo_e4m3_value.restype = C.c_double
        L.tqo_e4m3_encode.argtypes = [C.c_float]
        L.tqo_e4m3_encode.restype = C.c_uint8
        L.tqo_e2m1_nearest.argtypes = [C.c_float]
        L.tqo_e2m1_nearest.restype = i32
        L.tqo_e2m1_floor.argtypes = [C.c_float]
        L.tqo_e2m1_floor.restype = i32
        L.tqo_tensor_amax.argtypes = [p, i32, i64, i64, p]
        L.tqo_quantize.argtypes = [p, i32, i64, i64, i64, i32, p, p, p, p]
        L.tqo_quantize_guided.argtypes = [p, i32, i64, i64, i64, i32, p, p, p, p, p]
        L.tqo_extract_hint.argtypes = [p, i64, p]
        L.tqo_hint_first_layer.argtypes = [i32]
        L.tqo_hint_first_layer.restype = i32
        L.tqo_dequantize.argtypes = [p, p, p, i64, i64, i64, p]
        L.tqo_philox4x32_10.argtypes = [p, p, p]
        L.tqo_sr_byte.argtypes = [C.c_uint64, C.c_uint64]
        L.tqo_sr_byte.restype = i32
        L.tqo_sr_index.argtypes = [C.c_float, i32]
        L.tqo_sr_index.restype = i32
        L.tqo_requant_transpose_sr.argtypes = [p, p, p, i64, i64, i64, C.c_uint64, p, p, p, i64]
        L.tqo_grouped_gemm.argtypes = [p, p, C.c_int32, i64, i64, p, p, p, p, i64, p, p]
        L.tqo_e8m0_value.argtypes = [C.c_uint8]
        L.tqo_e8m0_value.restype = C.c_double
        L.tqo_e4m3_sr.argtypes = [C.c_float, i32]
        L.tqo_e4m3_sr.restype = i32
        L.tqo_quantize_mxfp8.argtypes = [p, i32, i64, i64, i64, p, p]
        L.tqo_requant_transpose_mxfp8_sr.argtypes = [p, p, p, i64, i64, i64, C.c_uint64, p, p, p, i64]
        L.tqo_quantize_tile16.argtypes = [p, i32, i64, i64, i64, i32, p, p, p, p]
        L.tqo_transpose_tile16.argtypes = [p, p, p, i64, i64, i64, p, p, p]
        L.tqo_grouped_gemm_w4a4.argtypes = [p, p, p, p, C.c_int32, i64, i64, p, p, p, p, i64, p, p]
        L.tqo_code_mismatch.argtypes = [p, p, i64, i64, p]
        L.tqo_e4m3_encode_array.argtypes = [p, i64, p]
        L.tqo_e2m1_nearest_array.argtypes = [p, i64, p]
        _lib = L
    return _lib


def _np(x, dtype=None):
    """numpy view of a CPU array or tensor; bf16 tensors become uint16 patterns."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                x = x.view(torch.int16).numpy().view(np.uint16)
            elif x.dtype == torch.uint8:
                x = x.numpy()
            else:
                x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if dtype is not None:
        assert x.dtype == dtype, (x.dtype, dtype)
    return x


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _x_and_dtype(x):
    a = _np(x)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"oracle input must be fp32 or bf16 (uint16 patterns), got {a.dtype}")


# ---- scalar format helpers ----------------------------------------------------------

def e2m1_value(code: int) -> float:
    return lib().tqo_e2m1_value(int(code))


def e4m3_value(b: int) -> float:
    return lib().tqo_e4m3_value(int(b))


def e4m3_encode(d: float) -> int:
    return int(lib().tqo_e4m3_encode(float(np.float32(d))))


def e2m1_nearest(a: float) -> int:
    return int(lib().tqo_e2m1_nearest(float(np.float32(a))))


def e2m1_floor(a: float) -> int:
    return int(lib().tqo_e2m1_floor(float(np.float32(a))))


def e4m3_encode_array(d):
    a = np.ascontiguousarray(np.asarray(d, np.float32))
    out = np.zeros(a.size, np.uint8)
    lib().tqo_e4m3_encode_array(_ptr(a), a.size, _ptr(out))
    return out


def e2m1_nearest_array(a):
    x = np.ascontiguousarray(np.asarray(a, np.float32))
    out = np.zeros(x.size, np.uint8)
    lib().tqo_e2m1_nearest_array(_ptr(x), x.size, _ptr(out))
    return out


def hint_first_layer(num_layers: int) -> int:
    return int(lib().tqo_hint_first_layer(int(num_layers)))


def sr_index(a: float, k: int) -> int:
    return int(lib().tqo_sr_index(float(np.float32(a)), int(k)))


# ---- tensor operations --------------------------------------------------------------

def tensor_amax(x, batch: int, per_tensor: int):
    a, dt = _x_and_dtype(x)
    out = np.zeros(batch, np.float32)
    lib().tqo_tensor_amax(_ptr(a), dt, batch, per_tensor, _ptr(out))
    return out


def _q_outputs(batch, rows, cols):
    n = batch * rows * cols
    return (np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), np.zeros(batch, np.float32))


def quantize(x, batch: int, rows: int, cols: int, amax=None):
    """Nearest quantizer Q.  Returns dict(codes, scales, tensor_scale, tensor_amax)."""
    a, dt = _x_and_dtype(x)
    assert a.size == batch * rows * cols and cols % 16 == 0
    codes, scales, ts = _q_outputs(batch, rows, cols)
    am = np.zeros(batch, np.float32) if amax is None else np.array(amax, np.float32).reshape(batch)
    lib().tqo_quantize(_ptr(a), dt, batch, rows, cols, 0 if amax is None else 1, _ptr(am),
                       _ptr(codes), _ptr(scales), _ptr(ts))
    return dict(codes=codes, scales=scales, tensor_scale=ts, tensor_amax=am)


def quantize_guided(x, batch: int, rows: int, cols: int, hints, amax=None):
    """Guided quantizer G (hints=None gives Q)."""
    a, dt = _x_and_dtype(x)
    assert a.size == batch * rows * cols and cols % 16 == 0
    codes, scales, ts = _q_outputs(batch, rows, cols)
    am = np.zeros(batch, np.float32) if amax is None else np.array(amax, np.float32).reshape(batch)
    h = None if hints is None else _np(hints, np.uint32)
    lib().tqo_quantize_guided(_ptr(a), dt, batch, rows, cols, 0 if amax is None else 1, _ptr(am),
                              None if h is None else _ptr(h), _ptr(codes), _ptr(scales), _ptr(ts))
    return dict(codes=codes, scales=scales, tensor_scale=ts, tensor_amax=am)


def extract_hint(codes, n: int):
    c = _np(codes, np.uint8)
    assert c.size * 2 >= n
    out = np.zeros((n + 31) // 32, np.uint32)
    lib().tqo_extract_hint(_ptr(c), n, _ptr(out))
    return out


def dequantize(codes, scales, tensor_scale, batch: int, rows: int, cols: int):
    c, s = _np(codes, np.uint8), _np(scales, np.uint8)
    t = _np(tensor_scale, np.float32)
    out = np.zeros(batch * rows * cols, np.float32)
    lib().tqo_dequantize(_ptr(c), _ptr(s), _ptr(t), batch, rows, cols, _ptr(out))
    return out


def philox4x32_10(ctr, key):
    c = np.array(ctr, np.uint32)
    k = np.array(key, np.uint32)
    out = np.zeros(4, np.uint32)
    lib().tqo_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_byte(seed: int, i: int) -> int:
    return int(lib().tqo_sr_byte(int(seed), int(i)))


def requant_transpose_sr(codes, scales, tensor_scale, batch: int, rows: int, cols: int, seed: int,
                         first: int = 0):
    """first: index of tensor 0 of this call within a larger batch (random-byte indices
    are those of the whole batch, outputs start at 0)."""
    c, s = _np(codes, np.uint8), _np(scales, np.uint8)
    t = _np(tensor_scale, np.float32)
    assert rows % 16 == 0 and cols % 16 == 0
    n = batch * rows * cols
    ct, st, tt = np.zeros(n // 2, np.uint8), np.zeros(n // 16, np.uint8), np.zeros(batch, np.float32)
    lib().tqo_requant_transpose_sr(_ptr(c), _ptr(s), _ptr(t), batch, rows, cols, int(seed),
                                   _ptr(ct), _ptr(st), _ptr(tt), int(first))
    return dict(codes=ct, scales=st, tensor_scale=tt)


def grouped_gemm(a, group_offsets, n: int, k: int, w_codes, w_scales, w_tensor_scale, rows=None):
    """fp64 reference rows of the grouped GEMM; returns (ref, abssum) of shape [len(rows), n]."""
    A = _np(a, np.uint16)
    off = _np(group_offsets, np.int32)
    wc, ws = _np(w_codes, np.uint8), _np(w_scales, np.uint8)
    wt = _np(w_tensor_scale, np.float32)
    m_total = A.size // k
    rows = np.arange(m_total, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    rows = np.ascontiguousarray(rows)
    ref = np.zeros((rows.size, n), np.float64)
    asum = np.zeros((rows.size, n), np.float64)
    lib().tqo_grouped_gemm(_ptr(A), _ptr(off), off.size - 1, n, k, _ptr(wc), _ptr(ws), _ptr(wt),
                           _ptr(rows), rows.size, _ptr(ref), _ptr(asum))
    return ref, asum


def e8m0_value(b: int) -> float:
    return lib().tqo_e8m0_value(int(b))


def e4m3_sr(a: float, k: int) -> int:
    return lib().tqo_e4m3_sr(float(a), int(k))


def quantize_mxfp8(x, batch: int, rows: int, cols: int):
    """Nearest MXFP8: codes [batch*rows*cols] E4M3 bytes, scales [batch*rows*cols/32] E8M0."""
    a, dt = _x_and_dtype(x)
    n = batch * rows * cols
    codes = np.zeros(n, np.uint8)
    scales = np.zeros(n // 32, np.uint8)
    lib().tqo_quantize_mxfp8(_ptr(a), dt, batch, rows, cols, _ptr(codes), _ptr(scales))
    return {"codes": codes, "scales": scales}


def requant_transpose_mxfp8_sr(codes, scales, tensor_scale, batch: int, rows: int, cols: int,
                               seed: int, first: int = 0):
    """NVFP4 [rows][cols] -> transposed MXFP8 [cols][rows] with stochastic rounding;
    `first` as in requant_transpose_sr."""
    c, s = _np(codes, np.uint8), _np(scales, np.uint8)
    ts = _np(tensor_scale, np.float32)
    n = batch * rows * cols
    ct = np.zeros(n, np.uint8)
    st = np.zeros(n // 32, np.uint8)
    tst = np.zeros(batch, np.float32)
    lib().tqo_requant_transpose_mxfp8_sr(_ptr(c), _ptr(s), _ptr(ts), batch, rows, cols,
                                         C.c_uint64(seed & (2 ** 64 - 1)), _ptr(ct), _ptr(st),
                                         _ptr(tst), int(first))
    return {"codes": ct, "scales": st, "tensor_scale": tst}


def quantize_tile16(x, batch: int, rows: int, cols: int, amax=None):
    """16x16-tile quantizer: codes [batch*rows*cols/2], scales [batch*(rows/16)*(cols/16)]."""
    a, dt = _x_and_dtype(x)
    n = batch * rows * cols
    codes = np.zeros(n // 2, np.uint8)
    scales = np.zeros(batch * (rows // 16) * (cols // 16), np.uint8)
    ts = np.zeros(batch, np.float32)
    am = np.zeros(batch, np.float32) if amax is None else np.ascontiguousarray(amax, np.float32).copy()
    lib().tqo_quantize_tile16(_ptr(a), dt, batch, rows, cols, int(amax is not None), _ptr(am),
                              _ptr(codes), _ptr(scales), _ptr(ts))
    return {"codes": codes, "scales": scales, "tensor_scale": ts, "tensor_amax": am}


def transpose_tile16(codes, scales, tensor_scale, batch: int, rows: int, cols: int):
    c, s = _np(codes, np.uint8), _np(scales, np.uint8)
    ts = _np(tensor_scale, np.float32)
    ct = np.zeros(c.size, np.uint8)
    st = np.zeros(s.size, np.uint8)
    tst = np.zeros(batch, np.float32)
    lib().tqo_transpose_tile16(_ptr(c), _ptr(s), _ptr(ts), batch, rows, cols, _ptr(ct), _ptr(st),
                               _ptr(tst))
    return {"codes": ct, "scales": st, "tensor_scale": tst}


def grouped_gemm_w4a4(a_codes, a_scales, a_tensor_scale, group_offsets, n: int, k: int, w_codes,
                      w_scales, w_tensor_scale, rows=None):
    """fp64 reference rows of the W4A4 grouped GEMM (activations one NVFP4 tensor
    [m_total][k]); returns (ref, abssum) of shape [len(rows), n]."""
    ac, as_ = _np(a_codes, np.uint8), _np(a_scales, np.uint8)
    at = _np(a_tensor_scale, np.float32)
    off = _np(group_offsets, np.int32)
    wc, ws = _np(w_codes, np.uint8), _np(w_scales, np.uint8)
    wt = _np(w_tensor_scale, np.float32)
    m_total = ac.size * 2 // k if k else 0
    rows = np.arange(m_total, dtype=np.int64) if rows is None else np.asarray(rows, np.int64)
    rows = np.ascontiguousarray(rows)
    ref = np.zeros((rows.size, n), np.float64)
    asum = np.zeros((rows.size, n), np.float64)
    lib().tqo_grouped_gemm_w4a4(_ptr(ac), _ptr(as_), _ptr(at), _ptr(off), off.size - 1, n, k,
                                _ptr(wc), _ptr(ws), _ptr(wt), _ptr(rows), rows.size, _ptr(ref),
                                _ptr(asum))
    return ref, asum


def code_mismatch(codes_a, codes_b, batch: int, per_tensor: int):
    a, b = _np(codes_a, np.uint8), _np(codes_b, np.uint8)
    out = np.zeros(2 * batch, np.uint64)
    lib().tqo_code_mismatch(_ptr(a), _ptr(b), batch, per_tensor, _ptr(out))
    return out.reshape(batch, 2)


def unpack_codes(codes, n: int):
    """4-bit codes, element 2j in the low nibble of byte j."""
    c = _np(codes, np.uint8)
    out = np.empty(c.size * 2, np.uint8)
    out[0::2] = c & 0x0F
    out[1::2] = c >> 4
    return out[:n]

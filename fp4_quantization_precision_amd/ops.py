"""Thin torch binding of libtq: argument marshalling only.

Every function takes torch tensors that live on the current HIP device, checks
their dtype, contiguity and device (so that no host pointer ever reaches a
kernel), and calls the C entry point of the same name on torch's current
stream.  All computation happens in the HIP kernels of libtq.so; a missing
library raises.  Nothing here synchronises.

Tensor conventions (see include/tq.h): bf16 inputs are torch.bfloat16, codes
and scales are torch.uint8, hint words are torch.int32 holding the uint32 bit
patterns, mismatch counters are torch.int64 holding uint64 counts.
"""
from __future__ import annotations

import ctypes as C
from typing import NamedTuple, Optional

import torch

from ._lib import TQ_AMAX_GIVEN, TQ_BF16, TQ_F32, check, lib

__all__ = [
    "NVFP4", "tensor_amax", "quantize", "quantize_guided", "extract_hint",
    "requant_transpose_sr", "grouped_gemm_nvfp4", "dequantize", "code_mismatch",
    "hint_first_layer", "hint_words", "new_nvfp4", "version",
]


class NVFP4(NamedTuple):
    """An NVFP4 tensor batch: codes [..., rows, cols/2], scales [..., rows, cols/16],
    tensor_scale [batch], plus the tensor amax it was made from."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    tensor_amax: torch.Tensor


def _need(t: torch.Tensor, name: str, dtypes) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return t


def _p(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _shape3(x: torch.Tensor):
    if x.dim() < 2:
        raise ValueError("expected at least 2 dims [..., rows, cols]")
    rows, cols = int(x.shape[-2]), int(x.shape[-1])
    batch = 1
    for s in x.shape[:-2]:
        batch *= int(s)
    return batch, rows, cols


def _dtype_code(x: torch.Tensor) -> int:
    return TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32


def hint_words(n: int) -> int:
    return (n + 31) // 32


def version() -> int:
    return int(lib().tq_version())


def hint_first_layer(num_layers: int) -> int:
    return int(lib().tq_hint_first_layer(int(num_layers)))


def new_nvfp4(batch_shape, rows: int, cols: int, device=None) -> NVFP4:
    """Uninitialised output buffers for a quantize call."""
    shape = tuple(batch_shape)
    batch = 1
    for s in shape:
        batch *= int(s)
    dev = device if device is not None else torch.device("cuda")
    return NVFP4(
        torch.empty(shape + (rows, cols // 2), dtype=torch.uint8, device=dev),
        torch.empty(shape + (rows, cols // 16), dtype=torch.uint8, device=dev),
        torch.empty(batch, dtype=torch.float32, device=dev),
        torch.empty(batch, dtype=torch.float32, device=dev),
    )


def tensor_amax(x: torch.Tensor, amax: Optional[torch.Tensor] = None, batch: Optional[int] = None):
    _need(x, "x", (torch.float32, torch.bfloat16))
    b = int(batch) if batch is not None else _shape3(x)[0]
    per = x.numel() // b if b else 0
    if amax is None:
        amax = torch.empty(b, dtype=torch.float32, device=x.device)
    _need(amax, "amax", (torch.float32,))
    check(lib().tq_tensor_amax(_p(x), _dtype_code(x), b, per, _p(amax), _stream()), "tq_tensor_amax")
    return amax


def _quantize(name, x, out: Optional[NVFP4], hints_in, hints_out, amax_given):
    _need(x, "x", (torch.float32, torch.bfloat16))
    batch, rows, cols = _shape3(x)
    if out is None:
        out = new_nvfp4(x.shape[:-2], rows, cols, x.device)
    _need(out.codes, "codes", (torch.uint8,))
    _need(out.scales, "scales", (torch.uint8,))
    _need(out.tensor_scale, "tensor_scale", (torch.float32,))
    _need(out.tensor_amax, "tensor_amax", (torch.float32,))
    n = batch * rows * cols
    if out.codes.numel() != n // 2 or out.scales.numel() != n // 16 or \
            out.tensor_scale.numel() != batch or out.tensor_amax.numel() != batch:
        raise ValueError("output buffers do not match the input shape")
    flags = TQ_AMAX_GIVEN if amax_given else 0
    hints = hints_in if hints_in is not None else hints_out
    if hints is not None:
        _need(hints, "hints", (torch.int32,))
        if hints.numel() < hint_words(n):
            raise ValueError("hint buffer too small")
    f = getattr(lib(), name)
    if name == "tq_quantize":
        st = f(_p(x), _dtype_code(x), batch, rows, cols, _p(out.tensor_amax), _p(out.codes),
               _p(out.scales), _p(out.tensor_scale), _p(hints_out), flags, _stream())
    else:
        st = f(_p(x), _dtype_code(x), batch, rows, cols, _p(out.tensor_amax), _p(hints_in),
               _p(out.codes), _p(out.scales), _p(out.tensor_scale), flags, _stream())
    check(st, name)
    return out


def quantize(x: torch.Tensor, out: Optional[NVFP4] = None, hints_out: Optional[torch.Tensor] = None,
             amax_given: bool = False) -> NVFP4:
    """Nearest NVFP4 quantization of x [..., rows, cols] (cols % 16 == 0).  With
    amax_given, out.tensor_amax is read instead of computed.  hints_out, if
    given, receives the packed 1-bit code parities."""
    return _quantize("tq_quantize", x, out, None, hints_out, amax_given)


def quantize_guided(x: torch.Tensor, hints: Optional[torch.Tensor], out: Optional[NVFP4] = None,
                    amax_given: bool = False) -> NVFP4:
    """Rollout-guided NVFP4 quantization of the trainer's x (hints=None: nearest)."""
    return _quantize("tq_quantize_guided", x, out, hints, None, amax_given)


def extract_hint(codes: torch.Tensor, n: int, hints: Optional[torch.Tensor] = None):
    _need(codes, "codes", (torch.uint8,))
    if codes.numel() * 2 < n:
        raise ValueError("codes too small for n")
    if hints is None:
        hints = torch.empty(hint_words(n), dtype=torch.int32, device=codes.device)
    _need(hints, "hints", (torch.int32,))
    if hints.numel() < hint_words(n):
        raise ValueError("hint buffer too small")
    check(lib().tq_extract_hint(_p(codes), int(n), _p(hints), _stream()), "tq_extract_hint")
    return hints


def requant_transpose_sr(q: NVFP4, batch: int, rows: int, cols: int, seed: int,
                         out: Optional[NVFP4] = None) -> NVFP4:
    """Dequantize -> transpose -> stochastic-rounding requantize of `batch`
    NVFP4 tensors of rows x cols; returns the cols x rows tensors."""
    _need(q.codes, "codes", (torch.uint8,))
    _need(q.scales, "scales", (torch.uint8,))
    _need(q.tensor_scale, "tensor_scale", (torch.float32,))
    n = batch * rows * cols
    if q.codes.numel() != n // 2 or q.scales.numel() != n // 16 or q.tensor_scale.numel() != batch:
        raise ValueError("input buffers do not match batch x rows x cols")
    if out is None:
        dev = q.codes.device
        out = NVFP4(torch.empty((batch, cols, rows // 2), dtype=torch.uint8, device=dev),
                    torch.empty((batch, cols, rows // 16), dtype=torch.uint8, device=dev),
                    torch.empty(batch, dtype=torch.float32, device=dev), q.tensor_amax)
    _need(out.codes, "codes_t", (torch.uint8,))
    _need(out.scales, "scales_t", (torch.uint8,))
    _need(out.tensor_scale, "tensor_scale_t", (torch.float32,))
    if out.codes.numel() != n // 2 or out.scales.numel() != n // 16 or \
            out.tensor_scale.numel() != batch:
        raise ValueError("output buffers do not match batch x cols x rows")
    check(lib().tq_requant_transpose_sr(_p(q.codes), _p(q.scales), _p(q.tensor_scale), batch, rows,
                                        cols, C.c_uint64(seed & (2 ** 64 - 1)), _p(out.codes),
                                        _p(out.scales), _p(out.tensor_scale), _stream()),
          "tq_requant_transpose_sr")
    return out


class MXFP8(NamedTuple):
    codes: torch.Tensor         # [..., rows, cols] E4M3 bytes
    scales: torch.Tensor        # [..., rows, cols/32] E8M0 bytes
    tensor_scale: Optional[torch.Tensor] = None  # carried by the transposed backward copy


def quantize_mxfp8(x: torch.Tensor) -> MXFP8:
    """Nearest MXFP8 of x [..., rows, cols] (cols % 32 == 0)."""
    _need(x, "x", (torch.float32, torch.bfloat16))
    cols = int(x.shape[-1])
    n = x.numel()
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty(tuple(x.shape[:-1]) + (cols // 32,), dtype=torch.uint8, device=x.device)
    dtype = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    rows = n // cols if cols else 0
    check(lib().tq_quantize_mxfp8(_p(x), dtype, 1, rows, cols, _p(codes), _p(scales), _stream()),
          "tq_quantize_mxfp8")
    return MXFP8(codes, scales)


def requant_transpose_mxfp8_sr(q: NVFP4, batch: int, rows: int, cols: int, seed: int) -> MXFP8:
    """NVFP4 [batch][rows][cols] -> transposed MXFP8 [batch][cols][rows] with
    stochastic rounding; the tensor scale is carried in the result."""
    _need(q.codes, "codes", (torch.uint8,))
    _need(q.scales, "scales", (torch.uint8,))
    _need(q.tensor_scale, "tensor_scale", (torch.float32,))
    n = batch * rows * cols
    if q.codes.numel() != n // 2 or q.scales.numel() != n // 16 or q.tensor_scale.numel() != batch:
        raise ValueError("input buffers do not match batch x rows x cols")
    dev = q.codes.device
    out = MXFP8(torch.empty((batch, cols, rows), dtype=torch.uint8, device=dev),
                torch.empty((batch, cols, rows // 32), dtype=torch.uint8, device=dev),
                torch.empty(batch, dtype=torch.float32, device=dev))
    check(lib().tq_requant_transpose_mxfp8_sr(_p(q.codes), _p(q.scales), _p(q.tensor_scale), batch,
                                              rows, cols, C.c_uint64(seed & (2 ** 64 - 1)),
                                              _p(out.codes), _p(out.scales), _p(out.tensor_scale),
                                              _stream()), "tq_requant_transpose_mxfp8_sr")
    return out


def quantize_tile16(x: torch.Tensor, amax_given: bool = False,
                    out: Optional[NVFP4] = None) -> NVFP4:
    """Nearest NVFP4 with one scale per 16x16 tile of x [..., rows, cols]; scales
    [..., rows/16, cols/16]."""
    _need(x, "x", (torch.float32, torch.bfloat16))
    if x.dim() < 2:
        raise ValueError("x must be [..., rows, cols]")
    rows, cols = int(x.shape[-2]), int(x.shape[-1])
    batch_shape = tuple(x.shape[:-2])
    batch = 1
    for d in batch_shape:
        batch *= int(d)
    if out is None:
        dev = x.device
        out = NVFP4(torch.empty(batch_shape + (rows, cols // 2), dtype=torch.uint8, device=dev),
                    torch.empty(batch_shape + (rows // 16, cols // 16), dtype=torch.uint8, device=dev),
                    torch.empty(batch, dtype=torch.float32, device=dev),
                    torch.empty(batch, dtype=torch.float32, device=dev))
    dtype = TQ_BF16 if x.dtype == torch.bfloat16 else TQ_F32
    check(lib().tq_quantize_tile16(_p(x), dtype, batch, rows, cols, _p(out.tensor_amax),
                                   _p(out.codes), _p(out.scales), _p(out.tensor_scale),
                                   TQ_AMAX_GIVEN if amax_given else 0, _stream()),
          "tq_quantize_tile16")
    return out


def transpose_tile16(q: NVFP4, batch: int, rows: int, cols: int,
                     out: Optional[NVFP4] = None) -> NVFP4:
    """Exact transpose of `batch` 16x16-tile NVFP4 tensors of rows x cols."""
    _need(q.codes, "codes", (torch.uint8,))
    _need(q.scales, "scales", (torch.uint8,))
    _need(q.tensor_scale, "tensor_scale", (torch.float32,))
    n = batch * rows * cols
    if q.codes.numel() != n // 2 or q.scales.numel() != n // 256 or q.tensor_scale.numel() != batch:
        raise ValueError("input buffers do not match batch x rows x cols")
    if out is None:
        dev = q.codes.device
        out = NVFP4(torch.empty((batch, cols, rows // 2), dtype=torch.uint8, device=dev),
                    torch.empty((batch, cols // 16, rows // 16), dtype=torch.uint8, device=dev),
                    torch.empty(batch, dtype=torch.float32, device=dev), q.tensor_amax)
    check(lib().tq_transpose_tile16(_p(q.codes), _p(q.scales), _p(q.tensor_scale), batch, rows,
                                    cols, _p(out.codes), _p(out.scales), _p(out.tensor_scale),
                                    _stream()), "tq_transpose_tile16")
    return out


def grouped_gemm_nvfp4(a: torch.Tensor, group_offsets: torch.Tensor, w: NVFP4, n: int, k: int,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[i] = bf16(s_e * a[i] @ W_e^T) for rows i of group e; W_e stored [n][k]."""
    _need(a, "a", (torch.bfloat16,))
    _need(group_offsets, "group_offsets", (torch.int32,))
    _need(w.codes, "w_codes", (torch.uint8,))
    _need(w.scales, "w_scales", (torch.uint8,))
    _need(w.tensor_scale, "w_tensor_scale", (torch.float32,))
    groups = group_offsets.numel() - 1
    m_total = a.numel() // k if k else int(a.shape[0])
    if a.numel() != m_total * k:
        raise ValueError("a must be [m_total, k]")
    if w.codes.numel() != groups * n * k // 2 or w.scales.numel() != groups * n * k // 16 or \
            w.tensor_scale.numel() != groups:
        raise ValueError("weights do not match groups x n x k")
    if out is None:
        out = torch.empty((m_total, n), dtype=torch.bfloat16, device=a.device)
    _need(out, "out", (torch.bfloat16,))
    if out.numel() != m_total * n:
        raise ValueError("out must be [m_total, n]")
    check(lib().tq_grouped_gemm_nvfp4(_p(a), _p(group_offsets), groups, m_total, n, k, _p(w.codes),
                                      _p(w.scales), _p(w.tensor_scale), _p(out), _stream()),
          "tq_grouped_gemm_nvfp4")
    return out


def grouped_gemm_w4a4(a: NVFP4, group_offsets: torch.Tensor, w: NVFP4, n: int, k: int,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[i] = bf16(s_a s_e * A~[i] @ W~_e^T) with the activations one NVFP4 tensor
    [m_total, k] (tq_quantize with batch 1) and W_e stored [n][k]."""
    for t, name in ((a.codes, "a_codes"), (a.scales, "a_scales"), (w.codes, "w_codes"),
                    (w.scales, "w_scales")):
        _need(t, name, (torch.uint8,))
    _need(a.tensor_scale, "a_tensor_scale", (torch.float32,))
    _need(w.tensor_scale, "w_tensor_scale", (torch.float32,))
    _need(group_offsets, "group_offsets", (torch.int32,))
    groups = group_offsets.numel() - 1
    m_total = a.codes.numel() * 2 // k if k else 0
    if a.codes.numel() * 2 != m_total * k or a.scales.numel() * 16 != m_total * k:
        raise ValueError("activations must be NVFP4 [m_total, k]")
    if w.codes.numel() != groups * n * k // 2 or w.scales.numel() != groups * n * k // 16 or \
            w.tensor_scale.numel() != groups:
        raise ValueError("weights do not match groups x n x k")
    if out is None:
        out = torch.empty((m_total, n), dtype=torch.bfloat16, device=a.codes.device)
    _need(out, "out", (torch.bfloat16,))
    if out.numel() != m_total * n:
        raise ValueError("out must be [m_total, n]")
    check(lib().tq_grouped_gemm_w4a4(_p(a.codes), _p(a.scales), _p(a.tensor_scale),
                                     _p(group_offsets), groups, m_total, n, k, _p(w.codes),
                                     _p(w.scales), _p(w.tensor_scale), _p(out), _stream()),
          "tq_grouped_gemm_w4a4")
    return out


def dequantize(q: NVFP4, batch: int, rows: int, cols: int, out: Optional[torch.Tensor] = None):
    _need(q.codes, "codes", (torch.uint8,))
    _need(q.scales, "scales", (torch.uint8,))
    _need(q.tensor_scale, "tensor_scale", (torch.float32,))
    if out is None:
        out = torch.empty((batch, rows, cols), dtype=torch.float32, device=q.codes.device)
    _need(out, "out", (torch.float32,))
    check(lib().tq_dequantize(_p(q.codes), _p(q.scales), _p(q.tensor_scale), batch, rows, cols,
                              _p(out), _stream()), "tq_dequantize")
    return out


def code_mismatch(codes_a: torch.Tensor, codes_b: torch.Tensor, batch: int, per_tensor: int,
                  counts: Optional[torch.Tensor] = None) -> torch.Tensor:
    """counts[t] = (#mismatched codes, #mismatches one signed grid step apart)."""
    _need(codes_a, "codes_a", (torch.uint8,))
    _need(codes_b, "codes_b", (torch.uint8,))
    if codes_a.numel() != batch * per_tensor // 2 or codes_b.numel() != codes_a.numel():
        raise ValueError("code arrays do not match batch x per_tensor")
    if counts is None:
        counts = torch.empty((batch, 2), dtype=torch.int64, device=codes_a.device)
    _need(counts, "counts", (torch.int64,))
    check(lib().tq_code_mismatch(_p(codes_a), _p(codes_b), batch, per_tensor, _p(counts),
                                 _stream()), "tq_code_mismatch")
    return counts

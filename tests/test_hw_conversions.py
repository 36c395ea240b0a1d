"""Device checks of the gfx950 conversions and arithmetic shortcuts the kernels rely on,
each over its whole input domain (tests/hw_conversions.hip, built by
__graft_entry__.build() into tests/libtq_hwcheck.so).  The references are written in
that file from the rules; a failure here means a kernel's shortcut no longer equals the
rule it stands for."""
import ctypes as C
import os

import pytest
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtq_hwcheck.so")

pytestmark = pytest.mark.gpu


def _run(name):
    assert os.path.exists(LIB), f"{LIB} is missing: run __graft_entry__.build()"
    lib = C.CDLL(LIB)
    fn = getattr(lib, name)
    fn.argtypes = [C.c_void_p, C.c_void_p]
    dev = torch.device("cuda")
    counts = torch.zeros(2, dtype=torch.int64, device=dev)
    first = torch.zeros(4, dtype=torch.int32, device=dev)
    print(f"\n{name}", flush=True)
    assert fn(C.c_void_p(counts.data_ptr()), C.c_void_p(first.data_ptr())) == 0
    f = [x & 0xFFFFFFFF for x in first.cpu().tolist()]
    return counts.cpu().tolist(), f


def test_fp4_nearest_every_binary32():
    """v_cvt_scalef32_pk_fp4_f32 (scale 1) is the E2M1 nearest rule (ties to the even
    index, 6 above 5) with the sign of x, for every finite binary32; the kernels then
    clear -0."""
    (bad, _), f = _run("hwc_fp4_nearest")
    assert bad == 0, f"input {f[1]:#010x}: got {f[2]:#x}, rule {f[3]:#x}"


def test_fp4_floor_every_binary32():
    """v_cvt_scalef32_sr_pk_fp4_f32 with a zero seed truncates |x| to the grid (6 and
    above give 6), sign kept: the floor the SR kernels and the guided quantizer use."""
    (bad, _), f = _run("hwc_fp4_floor")
    assert bad == 0, f"input {f[1]:#010x}: got {f[2]:#x}, rule {f[3]:#x}"


def test_fp4_decode_all_bytes():
    """v_cvt_scalef32_pk_f32_fp4 gives +-G[m] exactly for all 256 bytes, at scale 1 and
    at the power-of-two scale 2^-9 the SR kernel uses for its step sizes."""
    (bad, _), f = _run("hwc_fp4_decode")
    assert bad == 0, f"byte/scale {f[1]:#x}: got {f[2]:#010x}, rule {f[3]:#010x}"


def test_fp8_decode_all_byte_pairs():
    """v_cvt_scalef32_pk_f32_fp8 is the exact E4M3 decode for all 65536 byte pairs."""
    (bad, _), f = _run("hwc_fp8_decode")
    assert bad == 0, f"pair {f[1]:#06x}: got {f[2]:#010x} for byte {f[3]:#x}"


def test_fp8_nearest_every_binary32():
    """v_cvt_scalef32_pk_fp8_f32 (scale 1) is the E4M3 nearest rule (ties to the even
    code) with the sign of y for every finite |y| <= 464, and NaN above 464, where the
    rule saturates at 448: so the MXFP8 quantizer clamps to +-448 first and clears the
    sign of zero bytes."""
    (bad, big_not_nan), f = _run("hwc_fp8_nearest")
    assert bad == 0, f"input {f[1]:#010x}: got {f[2]:#x}, rule {f[3]:#x}"
    assert big_not_nan == 0


def test_div6_fast_path():
    """A * RN(1/6) with one FMA correction equals the correctly rounded A / 6 for A = 0
    and every finite A >= 2^-125 (the SR kernel's block maxima are 0 or >= 2^-10)."""
    (bad, _), f = _run("hwc_div6")
    assert bad == 0, f"A {f[1]:#010x}: got {f[2]:#010x}, correctly rounded {f[3]:#010x}"


def test_rcp_newton_e4m3():
    """v_rcp_f32 plus one Newton step equals the correctly rounded reciprocal of every
    nonzero finite E4M3 value (v_rcp_f32 alone misses some, which is why the step is
    there)."""
    (bad, rcp_alone_bad), f = _run("hwc_rcp_e4m3")
    assert bad == 0, f"byte {f[1]:#x}: got {f[2]:#010x}, correctly rounded {f[3]:#010x}"
    assert rcp_alone_bad > 0


def test_fp4_decode_f16_all_bytes():
    """v_cvt_scalef32_pk_f16_fp4 (scale 1) gives +-G[m] as binary16, -0 for the code of
    -0, for all 256 bytes in each byte position of its source word: the NVFP4 transpose
    stages its dequantized values in binary16."""
    (bad, _), f = _run("hwc_fp4_decode_f16")
    assert bad == 0, f"byte/position {f[1]:#x}: got {f[2]:#010x}, rule {f[3]:#010x}"


def test_fp8_decode_f16_all_byte_pairs():
    """v_cvt_scalef32_pk_f16_fp8 is the exact E4M3 decode into binary16 for all 65536
    byte pairs (every finite E4M3 value is a binary16 value)."""
    (bad, _), f = _run("hwc_fp8_decode_f16")
    assert bad == 0, f"pair {f[1]:#06x}: got {f[2]:#010x} for byte {f[3]:#x}"


def test_f16_scale_products_and_mixed_fma():
    """For every signed E2M1 code and E4M3 scale, the binary16 product G * dec is exact;
    and the mixed-precision FMA of that f16 value with each reciprocal the SR transpose
    uses (and 0) and a -0 addend is the binary32 product u * r, sign of zero included."""
    (bad, inexact), f = _run("hwc_f16_scale_products")
    assert inexact == 0, f"code/scale {f[1]:#x}: f16 product {f[2]:#010x} is not exact"
    assert bad == 0, f"case {f[1]:#x}: got {f[2]:#010x}, product {f[3]:#010x}"

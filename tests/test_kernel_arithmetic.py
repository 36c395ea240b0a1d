"""CPU checks of arithmetic reformulations that the HIP kernels rely on, each
against the rule it stands for, written here from that rule (no kernel and no
oracle code): the exactness of the dequantized products in the formats the
transpose kernels stage them in, and the 16-bit integer form of the MXFP8
stochastic rounding.  The kernels' results are checked bit for bit against the
oracle by the GPU parity tests; these tests pin the reasoning behind the
shortcuts over their whole domains."""
import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e4m3_values():
    """The 127 finite non-negative E4M3 values, by code 0x00 .. 0x7E."""
    out = []
    for b in range(0x7F):
        e, m = b >> 3, b & 7
        out.append(m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))
    return np.array(out)


def test_dequantized_products_exact_in_f16_and_bf16():
    """u = G[m] * dec(e) for every E2M1 magnitude and E4M3 scale: exact in binary16
    (the NVFP4 transpose's staging) and in bf16 (the MXFP8 transpose's staging), and
    zero or within [2^-10, 2688]."""
    u = (GRID[:, None] * e4m3_values()[None, :]).reshape(-1)
    assert np.array_equal(u.astype(np.float16).astype(np.float64), u)
    bf = (u.astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32).astype(np.float64)
    assert np.array_equal(bf, u)
    nz = u[u != 0]
    assert nz.min() == 2.0 ** -10 and nz.max() == 2688.0


def e4m3_sr_rule(y, k):
    """E4M3 stochastic rounding of y >= 0 (normal range or zero) with random byte k:
    the floor grid point lo, one step up iff k < 256 (y - lo) / spacing, 448 and above
    give the code 0x7E."""
    code = np.zeros(y.shape, np.int64)
    pos = y > 0
    e = np.floor(np.log2(np.where(pos, y, 1.0))).astype(np.int64)
    sp = np.ldexp(1.0, e - 3)
    lo = np.floor(np.where(pos, y, 0.0) / sp) * sp
    mant = np.round((lo / np.ldexp(1.0, e) - 1) * 8).astype(np.int64)
    lo_code = ((e + 7) << 3) | mant
    up = k < 256 * (y - lo) / sp
    code = np.where(pos, lo_code + up, 0)
    return np.where(y >= 448, 0x7E, np.minimum(code, 0x7E))


def test_mxfp8_sr_16bit_form_equals_the_rule():
    """For every bf16 magnitude pattern |u|16, every random byte k and shared exponents
    across the range: when y = |u| 2^-se is zero or at least 2^-6 (the fast path's
    condition), the code (min(max(|u|16 - K16, 0), 0x7E0) + 15 - (k >> 4)) >> 4 with
    K16 = (se + 120) << 7 equals the E4M3 rounding rule; and the fast-path test on the
    smallest nonzero pattern, (|u|16 - 1 mod 2^16) >= ((se + 121) << 7) - 1, holds
    exactly when every nonzero y is at least 2^-6."""
    a16 = np.arange(0x7F80, dtype=np.int64)  # finite magnitudes
    u = (a16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    k = np.arange(256, dtype=np.int64)
    for se in (-127, -100, -30, -9, -1, 0, 1, 7, 50, 120, 127):
        kexp = se + 120
        if kexp <= 0:
            continue
        y = np.ldexp(u, -se)
        ok = (y == 0) | (y >= 2.0 ** -6)
        # fast-path test, per pattern
        nz16 = (a16 - 1) % 65536
        assert np.array_equal((nz16 >= ((kexp + 1) << 7) - 1)[a16 != 0], ok[a16 != 0])
        a, yy = a16[ok], y[ok]
        x16 = np.minimum(np.maximum(a - (kexp << 7), 0), 0x7E0)
        got = (x16[:, None] + 15 - (k[None, :] >> 4)) >> 4
        want = e4m3_sr_rule(yy[:, None] * np.ones((1, 256)), k[None, :])
        assert np.array_equal(got, want), f"se {se}"

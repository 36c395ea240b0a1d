"""Pins of the CPU oracle against facts fixed independently of it.

Each test checks the oracle against something other than its own code: values
the pages print (golden fixtures with citations), an independent library
routine (torch's float8_e4m3fn cast, torch.matmul, ATen's Philox engine), an
independent formulation (per-binade round-half-even for E2M1), closed forms,
or invariants from the guided-rounding guarantee.  All run on the CPU.
"""
import json
import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def unpack(codes, n):
    c = np.asarray(codes, np.uint8).reshape(-1)
    out = np.empty(c.size * 2, np.uint8)
    out[0::2] = c & 0x0F
    out[1::2] = c >> 4
    return out[:n]


def pack(codes):
    c = np.asarray(codes, np.uint8)
    assert c.size % 2 == 0
    return (c[0::2] | (c[1::2] << 4)).astype(np.uint8)


def e4m3_torch(d):
    """torch's float8_e4m3fn cast (round to nearest even) of float32 values < 464."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(d, np.float32)))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_decode_torch(b):
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(b, np.uint8)))
    return t.view(torch.float8_e4m3fn).float().numpy()


def e2m1_rne_binade(a):
    """Independent E2M1 rounding: treat E2M1 as a mini-float with one mantissa
    bit; inside each binade the spacing is fixed (0.5 below 2, 1 in [2,4), 2 in
    [4,8)), so round-half-even of a/spacing gives the value; saturate at 6.
    Vectorised in float64, where a/spacing is exact."""
    a = np.asarray(a, np.float64)
    q = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    v = np.minimum(np.rint(a / q) * q, 6.0)  # np.rint: round half to even
    lut = {g: i for i, g in enumerate(GRID)}
    return np.array([lut[float(t)] for t in v], np.uint8)


def around(points, ulps=3):
    """Each float32 point and its neighbours up to `ulps` float32 ulps away."""
    out = []
    for p in points:
        x = np.float32(p)
        lo = hi = x
        out.append(x)
        for _ in range(ulps):
            lo = np.nextafter(lo, np.float32(-np.inf))
            hi = np.nextafter(hi, np.float32(np.inf))
            out += [lo, hi]
    out = np.array(out, np.float32)
    return out[out >= 0]


# ----------------------------------------------------------------------------------
# Number formats
# ----------------------------------------------------------------------------------

def test_e2m1_code_count_and_grid(orc):
    g = load("format_facts.json")
    vals = [orc.e2m1_value(c) for c in range(16)]
    assert len(vals) == g["codes_per_element"] == 16
    assert vals[:8] == g["e2m1_magnitudes"]
    assert vals[8:] == [-m for m in g["e2m1_magnitudes"]]
    assert len(set(vals)) == 15  # +0 and -0 coincide


def test_storage_is_4p5_bits_per_value(orc):
    g = load("format_facts.json")
    rows, cols = 8, 64
    x = np.random.default_rng(0).standard_normal(rows * cols).astype(np.float32)
    q = orc.quantize(x, 1, rows, cols)
    bits = 8.0 * (q["codes"].nbytes + q["scales"].nbytes) / (rows * cols)
    assert bits == g["bits_per_value_nvfp4"]
    assert cols // g["block_size"] == q["scales"].size // rows
    # The same arithmetic fixes MXFP8's 8.25 bits: one 8-bit scale per 32 values.
    assert 8 + 8 / 32 == g["bits_per_value_mxfp8"]
    assert 16 * 16 == g["tile_16x16_group"]


def test_e4m3_decode_matches_torch(orc):
    ours = np.array([orc.e4m3_value(b) for b in range(256)])
    ref = e4m3_decode_torch(np.arange(256)).astype(np.float64)
    nan = np.isnan(ref)
    assert nan.sum() == 2 and (np.isnan(ours) == nan).all()
    assert (ours[~nan] == ref[~nan]).all()
    assert orc.e4m3_value(0x7E) == 448.0 and orc.e4m3_value(0x01) == 2.0 ** -9


def test_e4m3_encode_matches_torch_dense(orc):
    finite = np.array(sorted({orc.e4m3_value(b) for b in range(0x7F)}), np.float64)
    mids = (finite[:-1] + finite[1:]) / 2
    pts = around(np.concatenate([finite, mids]), ulps=3)
    rng = np.random.default_rng(7)
    rand = np.exp2(rng.uniform(-14, np.log2(448.0), 300_000)).astype(np.float32)
    sub = rng.uniform(0, 2.0 ** -5, 100_000).astype(np.float32)
    d = np.concatenate([pts, rand, sub, np.float32([0.0, 2.0 ** -10, 2.0 ** -149])])
    d = d[(d >= 0) & (d < 448.0)]
    assert (orc.e4m3_encode_array(d) == e4m3_torch(d)).all()


def test_e4m3_encode_matches_torch_full_binade(orc):
    # every float32 in [1, 2): the rounding pattern of one whole binade
    bits = np.arange(0x3F800000, 0x40000000, dtype=np.uint32)
    d = bits.view(np.float32)
    assert (orc.e4m3_encode_array(d) == e4m3_torch(d)).all()


def test_e4m3_encode_saturates(orc):
    # reading: values at or above 448 saturate to the largest finite code
    for d in [448.0, 449.0, 463.9, 464.0, 480.0, 1e6, 3.0e38]:
        assert orc.e4m3_encode(d) == 0x7E
    assert orc.e4m3_encode(432.0) == 0x7E       # tie 416|448 goes to even mantissa
    assert orc.e4m3_encode(431.9) == 0x7D
    assert orc.e4m3_encode(2.0 ** -10) == 0x00  # tie 0|2^-9 goes to even code 0


def test_e2m1_nearest_matches_binade_rne(orc):
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    pts = around(mids + GRID + [6.5, 7.0, 8.0], ulps=3)
    rng = np.random.default_rng(3)
    a = np.concatenate([pts, rng.uniform(0, 8, 200_000).astype(np.float32),
                        np.float32([0.0, 1e-30, 1e30, 2.0 ** -149])])
    assert (orc.e2m1_nearest_array(a) == e2m1_rne_binade(a)).all()


def test_e2m1_nearest_full_binades(orc):
    # every float32 in [0.25, 8): all binades the E2M1 grid and its midpoints live in
    bits = np.arange(np.float32(0.25).view(np.uint32), np.float32(8.0).view(np.uint32),
                     dtype=np.uint32)
    a = bits.view(np.float32)
    ours = orc.e2m1_nearest_array(a)
    ref = e2m1_rne_binade(a[::97])  # python lut is slow: check a strided subset ...
    assert (ours[::97] == ref).all()
    # ... and the rest through the same rule, vectorised without the lookup
    q = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    v = np.minimum(np.rint(a.astype(np.float64) / q) * q, 6.0)
    grid = np.array(GRID)
    assert (grid[ours] == v).all()


def test_e2m1_floor(orc):
    for i, g in enumerate(GRID):
        assert orc.e2m1_floor(g) == i
        if i + 1 < len(GRID):
            assert orc.e2m1_floor(float(np.nextafter(np.float32(GRID[i + 1]), np.float32(0)))) == i
    assert orc.e2m1_floor(1e9) == 7


# ----------------------------------------------------------------------------------
# Q: nearest quantizer
# ----------------------------------------------------------------------------------

def _x_f32(x):
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    return x


def _block_views(x32, batch, rows, cols):
    return x32.reshape(batch, rows, cols // 16, 16)


def _random_tensor(kind, batch, rows, cols, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, rows, cols)).astype(np.float32)
    if kind == "outliers":
        m = rng.random(x.shape) < 0.002
        x[m] *= 40
    if kind == "mixed":
        x[:, :, :16] = 0.0                                  # zero blocks
        x[:, 1, 16:32] *= 2.0 ** -14                         # subnormal-scale blocks
        x[:, 2, 32:48] = -0.0                                # negative zero block
        x[0, 0, 48] = 1000.0                                 # one dominant value
    if kind == "bf16":
        t = torch.from_numpy(x * 0.02).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1)
    return x.reshape(-1)


CASES = [("plain", 1, 64, 256, 1), ("outliers", 3, 16, 128, 2), ("mixed", 2, 8, 64, 3),
         ("bf16", 4, 32, 96, 4)]


@pytest.mark.parametrize("kind,batch,rows,cols,seed", CASES)
def test_quantize_invariants(orc, kind, batch, rows, cols, seed):
    x = _random_tensor(kind, batch, rows, cols, seed)
    q = orc.quantize(x, batch, rows, cols)
    x32 = _x_f32(x).reshape(batch, rows, cols)
    codes = unpack(q["codes"], x.size).reshape(batch, rows, cols)
    scales = q["scales"].reshape(batch, rows, cols // 16)
    ts = q["tensor_scale"]

    # step 1: the tensor amax (numpy's max) and s_t = A_T / 2688
    A_T = np.abs(x32).reshape(batch, -1).max(axis=1)
    assert (q["tensor_amax"] == A_T).all()
    assert (ts == np.where(A_T == 0, 0, A_T / np.float32(2688))).all()

    dec = e4m3_decode_torch(scales).astype(np.float32)
    blocks = _block_views(x32, batch, rows, cols)
    A_b = np.abs(blocks).max(axis=3)
    for b in range(batch):
        if A_T[b] == 0:
            assert (scales[b] == 0).all() and (codes[b] == 0).all()
            continue
        # step 2: the scale byte is the E4M3 cast (torch) of (A_b / 6) / s_t
        d_b = (A_b[b] / np.float32(6)) / ts[b]
        assert (scales[b] == e4m3_torch(np.minimum(d_b, 448))).all()
        # the block holding the tensor maximum sits at the top of E4M3 (448)
        r, c = np.unravel_index(np.abs(x32[b]).argmax(), x32[b].shape)
        assert scales[b, r, c // 16] == 0x7E and (codes[b, r, c] & 7) == 7

        # step 3: each code is the nearest grid point of y = x * r_b (ties to even)
        S_b = dec[b] * ts[b]
        with np.errstate(divide="ignore", invalid="ignore"):
            r_b = np.float32(1) / S_b
            y = blocks[b] * r_b[..., None]
        live = np.broadcast_to((dec[b] != 0)[..., None], y.shape)
        m = (codes[b].reshape(y.shape) & 7).astype(np.int64)
        sgn = (codes[b].reshape(y.shape) >> 3).astype(np.int64)
        assert (codes[b].reshape(y.shape)[~live] == 0).all()
        a = np.abs(y[live]).astype(np.float64)
        mm = m[live]
        dist = np.abs(a[:, None] - np.array(GRID)[None, :])
        best = dist.min(axis=1)
        assert (dist[np.arange(a.size), mm] == best).all()
        tie = (dist == best[:, None]).sum(axis=1) > 1
        assert (mm[tie] % 2 == 0).all()
        # sign: set exactly for negative y with a nonzero magnitude (zero is +0)
        assert ((sgn[live] == 1) == ((y[live] < 0) & (mm != 0))).all()

        # scale convention: in blocks with a normal E4M3 scale, max|y| is 6 up to
        # the scale's 2^-4 relative rounding
        normal = scales[b] >= 8
        ymax = np.abs(y).max(axis=2)[normal]
        assert (ymax >= 6 / (1 + 2.0 ** -4) * (1 - 1e-6)).all()
        assert (ymax <= 6 * (1 + 2.0 ** -4) * (1 + 1e-6)).all()

    # dequantised values are within one grid half-gap (<= 1) of y, in x units
    v = orc.dequantize(q["codes"], q["scales"], ts, batch, rows, cols).reshape(batch, rows, cols)
    S = (dec * ts[:, None, None])
    S_full = np.repeat(S, 16, axis=2)
    normal_full = np.repeat(scales >= 8, 16, axis=2)
    err = np.abs(x32.astype(np.float64) - v)
    bound = S_full.astype(np.float64) * 1.0 * (1 + 1e-6) + 1e-6 * np.abs(x32)
    assert (err[normal_full] <= bound[normal_full]).all()


def test_quantize_all_zero_and_empty_tensors(orc):
    x = np.zeros(2 * 16 * 32, np.float32)
    x[16 * 32:] = -0.0
    q = orc.quantize(x, 2, 16, 32)
    assert (q["codes"] == 0).all() and (q["scales"] == 0).all()
    assert (q["tensor_scale"] == 0).all() and (q["tensor_amax"] == 0).all()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_tensor_amax_matches_numpy(orc, dtype):
    """The oracle's per-tensor amax against numpy's max |x| per tensor of a batch:
    random tensors of mixed magnitudes, a tensor whose maximum is negative, one of
    subnormals only, one of signed zeros, and single-block tensors."""
    rng = np.random.default_rng(21)
    shapes = [(7, 48), (3, 4096), (1, 16), (5, 16 * 65)]
    for batch, per in shapes:
        x = (rng.standard_normal((batch, per)) *
             np.exp2(rng.uniform(-40, 40, (batch, 1)))).astype(np.float32)
        x[0] = -np.abs(x[0])                                       # maximum |x| at a negative value
        if batch > 2:
            x[1] = (rng.standard_normal(per) * 1e-39).astype(np.float32)  # subnormals only
            x[2] = np.where(rng.random(per) < 0.5, -0.0, 0.0).astype(np.float32)
        if dtype == "bf16":
            t = torch.from_numpy(x).to(torch.bfloat16)
            want = t.float().abs().amax(dim=1).numpy()
            got = orc.tensor_amax(t.view(torch.int16).numpy().view(np.uint16), batch, per)
        else:
            want = np.abs(x).max(axis=1)
            got = orc.tensor_amax(x, batch, per)
        assert np.array_equal(got, want.astype(np.float32)), (batch, per)


def test_quantize_amax_given_matches_computed(orc):
    x = _random_tensor("outliers", 3, 16, 128, 9)
    q1 = orc.quantize(x, 3, 16, 128)
    q2 = orc.quantize(x, 3, 16, 128, amax=q1["tensor_amax"])
    for k in ("codes", "scales", "tensor_scale"):
        assert (q1[k] == q2[k]).all()


def test_boundary_example_from_trace_page(orc):
    """TRACE explainer, rounding-boundary analogy: values either side of 2.5
    round to different bins; the rollout's bin, sent as a 1-bit hint, pulls the
    training side over.  Unit scale: A_T = 2688 gives s_t = 1, and a block whose
    maximum is 6 gets block scale 1, so y equals x."""
    g = load("rounding_boundary.json")
    xr = np.zeros(32, np.float32)
    xt = np.zeros(32, np.float32)
    xr[0] = xt[0] = 6.0
    xr[16] = xt[16] = 2688.0
    xr[1], xt[1] = g["rollout_value"], g["train_value"]
    qr = orc.quantize(xr, 1, 1, 32)
    qt = orc.quantize(xt, 1, 1, 32)
    assert qr["tensor_scale"][0] == 1.0 and qr["scales"][0] == 0x38
    cr, ct = unpack(qr["codes"], 32), unpack(qt["codes"], 32)
    assert cr[1] == g["rollout_nearest_code"] and ct[1] == g["train_nearest_code"]
    h = orc.extract_hint(qr["codes"], 32)
    assert (h[0] >> 1) & 1 == g["hint_bit"]
    qg = orc.quantize_guided(xt, 1, 1, 32, h)
    assert unpack(qg["codes"], 32)[1] == g["train_guided_code"]


# ----------------------------------------------------------------------------------
# H: hints and layer gating
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [0, 1, 2, 31, 32, 33, 64, 1000, 4096 + 16])
def test_hint_is_packed_code_parity(orc, n):
    rng = np.random.default_rng(n)
    codes = rng.integers(0, 256, (n + 1) // 2, dtype=np.uint8)
    h = orc.extract_hint(codes, n)
    assert h.size == (n + 31) // 32
    parity = unpack(codes, n) & 1
    ref = np.packbits(parity, bitorder="little")
    ref = np.concatenate([ref, np.zeros((-ref.size) % 4, np.uint8)]).view("<u4")
    assert (h == ref).all()


def test_layer_gating(orc):
    for L, first in load("layer_gating.json")["cases"]:
        assert orc.hint_first_layer(L) == first


# ----------------------------------------------------------------------------------
# G: guided quantizer and its guarantee
# ----------------------------------------------------------------------------------

def _bracket(v):
    """Indices allowed for the guided code of value v at unit scale: the grid
    point itself when v is on the grid, else the two points around |v|; 7 for
    |v| >= 6.  Exact, with Fractions."""
    a = abs(Fraction(float(v)))
    if a >= 6:
        return {7}
    grid = [Fraction(g) for g in GRID]
    if a in grid:
        return {grid.index(a)}
    lo = max(i for i, g in enumerate(grid) if g <= a)
    return {lo, lo + 1}


def _signed(m, v):
    return m | (8 if (v < 0 and m != 0) else 0)


def _unit_scale_blocks(values):
    """Pack values into rows of [6, v0..v14] blocks plus one 2688 sentinel
    block, so s_t = 1 and each value block has scale 1 (y = x)."""
    per = 15
    nb = (len(values) + per - 1) // per
    cols = 16 * (nb + 1)
    x = np.zeros(cols, np.float32)
    pos = []
    for i, v in enumerate(values):
        blk, j = divmod(i, per)
        x[16 * blk] = 6.0
        x[16 * blk + 1 + j] = v
        pos.append(16 * blk + 1 + j)
    x[16 * nb] = 2688.0
    return x, np.array(pos), cols


def test_guided_guarantee_bruteforce(orc):
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    base = list(around(mids + GRID + [6.2], ulps=1)) + [0.1, 0.4, 0.6, 1.1, 2.2, 2.9, 4.5, 5.5]
    vals = sorted(set(float(v) for v in base))
    vals = vals + [-v for v in vals if v != 0]
    pairs = [(r, t) for r in vals for t in vals]
    xr_vals = [p[0] for p in pairs]
    xt_vals = [p[1] for p in pairs]
    xr, pos, cols = _unit_scale_blocks(xr_vals)
    xt, _, _ = _unit_scale_blocks(xt_vals)
    qr = orc.quantize(xr, 1, 1, cols)
    qn = orc.quantize(xt, 1, 1, cols)
    h = orc.extract_hint(qr["codes"], cols)
    qg = orc.quantize_guided(xt, 1, 1, cols, h)
    assert qr["tensor_scale"][0] == 1.0
    r = unpack(qr["codes"], cols)[pos]
    n = unpack(qn["codes"], cols)[pos]
    g = unpack(qg["codes"], cols)[pos]
    mism_g = mism_n = expected_g = 0
    for i, (vr, vt) in enumerate(pairs):
        allowed = {_signed(m, vt) for m in _bracket(vt)}
        assert g[i] in allowed and n[i] in allowed
        in_bracket = r[i] in allowed
        assert (g[i] == r[i]) == in_bracket
        mism_g += int(g[i] != r[i])
        mism_n += int(n[i] != r[i])
        expected_g += int(not in_bracket)
    assert mism_g == expected_g <= mism_n
    assert mism_n > mism_g  # the boundary cases are in the set


def test_guided_special_cases(orc):
    x = _random_tensor("bf16", 2, 16, 64, 21)
    q = orc.quantize(x, 2, 16, 64)
    h_self = orc.extract_hint(q["codes"], x.size)
    # hints taken from the tensor's own nearest codes reproduce Q exactly
    g = orc.quantize_guided(x, 2, 16, 64, h_self)
    assert (g["codes"] == q["codes"]).all() and (g["scales"] == q["scales"]).all()
    # no hints: identical to Q
    g0 = orc.quantize_guided(x, 2, 16, 64, None)
    assert (g0["codes"] == q["codes"]).all()
    # arbitrary hints never move a code off the bracket nor change the scales
    rng = np.random.default_rng(5)
    h_rand = rng.integers(0, 2 ** 32, h_self.size, dtype=np.uint64).astype(np.uint32)
    gr = orc.quantize_guided(x, 2, 16, 64, h_rand)
    assert (gr["scales"] == q["scales"]).all()
    cq, cg = unpack(q["codes"], x.size), unpack(gr["codes"], x.size)
    dq = np.where(cq & 8, -1, 1) * (cq & 7).astype(int)
    dg = np.where(cg & 8, -1, 1) * (cg & 7).astype(int)
    assert (np.abs(dq - dg) <= 1).all()


# ----------------------------------------------------------------------------------
# Philox4x32-10
# ----------------------------------------------------------------------------------

def test_philox_known_answers(orc):
    for v in load("philox_kat.json")["vectors"]:
        ctr = [int(c, 16) for c in v["counter"]]
        key = [int(k, 16) for k in v["key"]]
        out = [int(o, 16) for o in v["out"]]
        assert list(orc.philox4x32_10(ctr, key)) == out


ATEN_XCHECK = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned c0, c1, c2, c3, k0, k1;
  while (std::scanf("%x %x %x %x %x %x", &c0, &c1, &c2, &c3, &k0, &k1) == 6) {
    unsigned long long seed = ((unsigned long long)k1 << 32) | k0;
    unsigned long long sub = ((unsigned long long)c3 << 32) | c2;
    unsigned long long off = ((unsigned long long)c1 << 32) | c0;
    at::philox_engine e(seed, sub, off);
    unsigned w0 = e(), w1 = e(), w2 = e(), w3 = e();
    std::printf("%08x %08x %08x %08x\n", w0, w1, w2, w3);
  }
}
"""


def test_philox_matches_aten_engine(orc, tmp_path):
    """ATen's header-only Philox4x32-10 engine is an independent implementation;
    it is compiled here into a throwaway test binary only."""
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    src = tmp_path / "x.cpp"
    src.write_text(ATEN_XCHECK)
    exe = tmp_path / "x"
    subprocess.run(["g++", "-std=c++17", "-O1", f"-I{inc}", str(src), "-o", str(exe)], check=True)
    rng = np.random.default_rng(11)
    rows = rng.integers(0, 2 ** 32, (400, 6), dtype=np.uint64).astype(np.uint32)
    rows[:50, 1:4] = 0  # counters of the form used by the transpose step
    text = "\n".join(" ".join(f"{v:08x}" for v in r) for r in rows) + "\n"
    res = subprocess.run([str(exe)], input=text, capture_output=True, text=True, check=True)
    got = [[int(t, 16) for t in line.split()] for line in res.stdout.strip().splitlines()]
    for r, w in zip(rows, got):
        assert list(orc.philox4x32_10(r[:4], r[4:])) == w


def test_sr_byte_layout(orc):
    # byte i mod 16 of the block's four words, little-endian
    seed = 0x0123456789ABCDEF
    for beta in [0, 1, 77, 2 ** 32 + 5]:
        w = orc.philox4x32_10([beta & 0xFFFFFFFF, beta >> 32, 0, 0],
                              [seed & 0xFFFFFFFF, seed >> 32])
        raw = np.array(w, "<u4").view(np.uint8)
        for j in range(16):
            assert orc.sr_byte(seed, 16 * beta + j) == raw[j]


# ----------------------------------------------------------------------------------
# S: transpose-requantize with stochastic rounding
# ----------------------------------------------------------------------------------

def test_sr_example_from_tml_page(orc):
    """TML article: 2.25 goes to 2 three times in four and to 3 once; the mean
    stays 2.25.  With 8 random bits exactly 64 of the 256 bytes round up."""
    g = load("sr_example.json")
    ups = [orc.sr_index(g["value"], k) for k in range(256)]
    lo_i, hi_i = GRID.index(g["lower"]), GRID.index(g["upper"])
    assert set(ups) == {lo_i, hi_i}
    assert ups.count(hi_i) == 256 * g["p_upper"] == 64
    mean = sum(GRID[m] for m in ups) / 256
    assert mean == g["mean"]


def _sr_input_225(cols=16):
    """16 x cols NVFP4 tensor whose column 0 dequantises to [6, 2.25 x 15]:
    row 0 holds G=6 at block scale 1 (0x38), rows 1..15 hold G=1.5 at block
    scale 1.5 (0x3C); so the new block has max 6, scale 1, and y = u."""
    codes = np.zeros((16, cols), np.uint8)
    scales = np.full((16, cols // 16), 0x38, np.uint8)
    codes[0, 0] = 7
    codes[1:, 0] = 3
    scales[1:, 0] = 0x3C
    return pack(codes.reshape(-1)), scales.reshape(-1), np.float32([1.0])


def test_sr_example_through_transpose(orc):
    g = load("sr_example.json")
    codes, scales, ts = _sr_input_225()
    ups = 0
    seeds = 2048
    for seed in range(seeds):
        out = orc.requant_transpose_sr(codes, scales, ts, 1, 16, 16, seed)
        assert out["scales"][0] == 0x38 and out["tensor_scale"][0] == 1.0
        row0 = unpack(out["codes"], 256)[:16]
        assert row0[0] == 7
        assert set(row0[1:].tolist()) <= {4, 5}
        ups += int((row0[1:] == 5).sum())
    n = 15 * seeds
    p = ups / n
    sigma = (g["p_upper"] * g["p_lower"] / n) ** 0.5
    assert abs(p - g["p_upper"]) < 5 * sigma


def test_sr_on_grid_is_exact_transpose(orc):
    """When every new block's maximum is 6 at unit scales, all y lie on the grid
    and the step reduces to a plain transpose of the codes (-0 becomes +0)."""
    rng = np.random.default_rng(13)
    R, Cc, B = 48, 64, 2
    codes = rng.integers(0, 16, (B, R, Cc), dtype=np.uint8)
    codes[:, ::16, :] = rng.choice([7, 15], (B, R // 16, Cc))
    scales = np.full((B, R, Cc // 16), 0x38, np.uint8)
    ts = np.float32([0.25, 3.0])
    out = orc.requant_transpose_sr(pack(codes.reshape(-1)), scales.reshape(-1), ts, B, R, Cc, 99)
    got = unpack(out["codes"], B * R * Cc).reshape(B, Cc, R)
    want = codes.transpose(0, 2, 1).copy()
    want[want == 8] = 0
    assert (got == want).all()
    assert (out["scales"] == 0x38).all() and (out["tensor_scale"] == ts).all()
    # and the dequantised tensor is the transpose of the dequantised input
    dq_in = orc.dequantize(pack(codes.reshape(-1)), scales.reshape(-1), ts, B, R, Cc)
    dq_out = orc.dequantize(out["codes"], out["scales"], ts, B, Cc, R)
    assert (dq_out.reshape(B, Cc, R) == dq_in.reshape(B, R, Cc).transpose(0, 2, 1)).all()


def test_sr_first_tensor_offset(orc):
    """One tensor of a batch recomputed alone: with `first` = its index the random
    bytes are those of the whole batch, so both transposes reproduce that tensor's
    slice of the batch output (and differ from a call without the offset)."""
    from fp4_quantization_precision_amd import inputs
    B, R, Cc, b = 3, 64, 48, 2
    c, s, ts = (t.numpy().reshape(-1) for t in inputs.random_nvfp4(B, R, Cc, seed=23))
    per = R * Cc
    cb, sb, tb = c[b * per // 2:(b + 1) * per // 2], s[b * per // 16:(b + 1) * per // 16], ts[b:b + 1]
    full = orc.requant_transpose_sr(c, s, ts, B, R, Cc, 5)
    one = orc.requant_transpose_sr(cb, sb, tb, 1, R, Cc, 5, first=b)
    assert np.array_equal(one["codes"], full["codes"][b * per // 2:(b + 1) * per // 2])
    assert np.array_equal(one["scales"], full["scales"][b * per // 16:(b + 1) * per // 16])
    assert not np.array_equal(one["codes"], orc.requant_transpose_sr(cb, sb, tb, 1, R, Cc, 5)["codes"])
    full = orc.requant_transpose_mxfp8_sr(c, s, ts, B, R, Cc, 5)
    one = orc.requant_transpose_mxfp8_sr(cb, sb, tb, 1, R, Cc, 5, first=b)
    assert np.array_equal(one["codes"], full["codes"][b * per:(b + 1) * per])
    assert np.array_equal(one["scales"], full["scales"][b * per // 32:(b + 1) * per // 32])
    assert not np.array_equal(one["codes"],
                              orc.requant_transpose_mxfp8_sr(cb, sb, tb, 1, R, Cc, 5)["codes"])


def test_sr_bracket_and_bias(orc):
    """Random stored tensors (zero blocks included): every output code lies in
    the bracket of y = u * r' (exact check with the torch E4M3 cast of A'/6),
    and over 64 seeds the mean of the rounded values matches y up to the
    8-bit resolution of the random bytes."""
    from fp4_quantization_precision_amd import inputs
    B, R, Cc = 1, 32, 64
    c, s, ts = inputs.random_nvfp4(B, R, Cc, seed=3, zero_block_frac=0.1)
    c, s, ts = c.numpy(), s.numpy(), ts.numpy()
    codes = unpack(c, B * R * Cc).reshape(R, Cc)
    dec = e4m3_decode_torch(s).astype(np.float64).reshape(R, Cc // 16)
    u = np.array(GRID)[codes & 7] * np.repeat(dec, 16, axis=1) * np.where(codes & 8, -1, 1)
    uT = u.T.astype(np.float32)                         # [Cc][R], exact in float32
    A = np.abs(uT).reshape(Cc, R // 16, 16).max(axis=2)
    e_new = e4m3_torch(np.minimum(A / np.float32(6), 448))
    dnew = e4m3_decode_torch(e_new).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        rr = np.float32(1) / dnew
        y = (uT.reshape(Cc, R // 16, 16) * rr[..., None]).reshape(Cc, R)
    live = np.repeat(dnew != 0, 16, axis=1)
    a = np.abs(y[live]).astype(np.float64)
    grid = np.array(GRID)
    lo = np.searchsorted(grid, a, side="right") - 1
    hi = np.minimum(lo + 1, 7)
    on = (grid[lo] == a) | (a >= 6)   # a >= 6 saturates to index 7 deterministically
    acc = np.zeros(a.size)
    S = 64
    for seed in range(S):
        out = orc.requant_transpose_sr(c, s, ts, B, R, Cc, seed)
        assert (out["scales"] == e_new.reshape(-1)).all()
        oc = unpack(out["codes"], B * R * Cc).reshape(Cc, R)
        assert (oc[~live] == 0).all()
        m = (oc[live] & 7).astype(np.int64)
        ok = np.where(on, m == lo, (m == lo) | (m == hi))
        assert ok.all()
        sign_ok = ((oc[live] >> 3) == 1) == ((y[live] < 0) & (m != 0))
        assert sign_ok.all()
        acc += grid[m]
    mean = acc / S
    delta = grid[hi] - grid[lo]
    p = np.where(on, 0, (a - grid[lo]) / np.where(delta == 0, 1, delta))
    # 8-bit rule: P(up) = ceil(256 p) / 256, so the expected bias lies in [0, delta/256)
    q = np.ceil(256 * p) / 256
    expect = np.where(a >= 6, 6.0, grid[lo] + delta * q)
    sd = delta * np.sqrt(q * (1 - q) / S)
    z = np.abs(mean - expect) / np.where(sd == 0, 1, sd)
    assert (np.abs(mean - expect)[sd == 0] == 0).all()
    assert (z < 6).all()
    inb = a < 6
    assert ((expect - a)[inb] >= 0).all() and ((expect - a)[inb] < delta[inb] / 256 + 1e-12).all()
    # globally the stochastic rounding keeps the mean (the TML page's point)
    inner = a < 6
    tot_sd = np.sqrt(np.sum(sd[inner] ** 2)) / inner.sum()
    bias = np.mean((mean - a)[inner])
    assert -5 * tot_sd <= bias <= np.mean(delta[inner]) / 256 + 5 * tot_sd


# ----------------------------------------------------------------------------------
# M: grouped GEMM reference
# ----------------------------------------------------------------------------------

def _w_values(wc, ws, wts, E, n, k):
    codes = unpack(wc, E * n * k).reshape(E, n, k)
    dec = e4m3_decode_torch(ws).astype(np.float64).reshape(E, n, k // 16)
    return (np.array(GRID)[codes & 7] * np.where(codes & 8, -1.0, 1.0)
            * np.repeat(dec, 16, axis=2) * wts.astype(np.float64)[:, None, None])


def test_gemm_oracle_matches_torch_matmul(orc):
    rng = np.random.default_rng(17)
    counts = [5, 0, 7, 1]
    E, n, k = len(counts), 24, 48
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    a = torch.from_numpy(rng.standard_normal((M, k)).astype(np.float32)).to(torch.bfloat16)
    wc = rng.integers(0, 256, E * n * k // 2, dtype=np.uint8)
    ws = rng.integers(0, 0x7F, E * n * k // 16, dtype=np.uint8)
    wts = rng.uniform(0.1, 2.0, E).astype(np.float32)
    ref, asum = orc.grouped_gemm(a, off, n, k, wc, ws, wts)
    W = torch.from_numpy(_w_values(wc, ws, wts, E, n, k))
    A = a.double()
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        want = torch.matmul(A[lo:hi], W[e].T).numpy()
        wabs = torch.matmul(A[lo:hi].abs(), W[e].T.abs()).numpy()
        assert np.allclose(ref[lo:hi], want, rtol=0, atol=1e-12 * max(1.0, wabs.max()))
        assert np.allclose(asum[lo:hi], wabs, rtol=1e-12, atol=0)


def test_gemm_oracle_closed_form(orc):
    # W = 1 everywhere (code 2 = 1.0, scale 0x38 = 1.0, tensor scale 1) -> row sums
    E, n, k = 2, 8, 32
    off = np.array([0, 3, 5], np.int32)
    A = np.arange(5 * k, dtype=np.float32).reshape(5, k) % 7 - 3
    a = torch.from_numpy(A).to(torch.bfloat16)
    wc = np.full(E * n * k // 2, 0x22, np.uint8)
    ws = np.full(E * n * k // 16, 0x38, np.uint8)
    wts = np.float32([1.0, 0.5])
    ref, asum = orc.grouped_gemm(a, off, n, k, wc, ws, wts, rows=[0, 2, 3, 4])
    rows = A[[0, 2, 3, 4]].sum(axis=1)
    scale = np.array([1.0, 1.0, 0.5, 0.5])
    assert (ref == (rows * scale)[:, None]).all()
    assert (asum == (np.abs(A[[0, 2, 3, 4]]).sum(axis=1) * scale)[:, None]).all()


def test_w4a4_gemm_oracle_matches_torch_matmul(orc):
    """Activations NVFP4 too: the oracle equals a float64 matmul of both operands
    decoded independently here (grid table x torch's E4M3 decode x tensor scale)."""
    rng = np.random.default_rng(23)
    counts = [3, 0, 9, 4]
    E, n, k = len(counts), 16, 64
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    ac = rng.integers(0, 256, M * k // 2, dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, M * k // 16, dtype=np.uint8)
    at = np.float32([0.37])
    wc = rng.integers(0, 256, E * n * k // 2, dtype=np.uint8)
    ws = rng.integers(0, 0x7F, E * n * k // 16, dtype=np.uint8)
    wts = rng.uniform(0.1, 2.0, E).astype(np.float32)
    ref, asum = orc.grouped_gemm_w4a4(ac, as_, at, off, n, k, wc, ws, wts)
    A = torch.from_numpy(_w_values(ac, as_, at, 1, M, k)[0])
    W = torch.from_numpy(_w_values(wc, ws, wts, E, n, k))
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        want = torch.matmul(A[lo:hi], W[e].T).numpy()
        wabs = torch.matmul(A[lo:hi].abs(), W[e].T.abs()).numpy()
        assert np.allclose(ref[lo:hi], want, rtol=0, atol=1e-12 * max(1.0, wabs.max()))
        assert np.allclose(asum[lo:hi], wabs, rtol=1e-12, atol=0)


def test_w4a4_gemm_reduces_to_w4a16(orc):
    """With a power-of-two activation tensor scale every dequantized activation is
    exact in bf16, so the W4A4 result equals the (pinned) bf16-activation GEMM on
    those bf16 values, bit for bit."""
    rng = np.random.default_rng(29)
    counts = [6, 2, 0, 5]
    E, n, k = len(counts), 8, 48
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(off[-1])
    ac = rng.integers(0, 256, M * k // 2, dtype=np.uint8)
    as_ = rng.integers(0, 0x7F, M * k // 16, dtype=np.uint8)
    at = np.float32([0.25])
    wc = rng.integers(0, 256, E * n * k // 2, dtype=np.uint8)
    ws = rng.integers(0, 0x7F, E * n * k // 16, dtype=np.uint8)
    wts = rng.uniform(0.1, 2.0, E).astype(np.float32)
    A = _w_values(ac, as_, at, 1, M, k)[0]
    a_bf16 = torch.from_numpy(A.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(a_bf16.double().numpy(), A)  # exact in bf16
    ref4, asum4 = orc.grouped_gemm_w4a4(ac, as_, at, off, n, k, wc, ws, wts)
    ref16, asum16 = orc.grouped_gemm(a_bf16, off, n, k, wc, ws, wts)
    assert np.array_equal(ref4, ref16) and np.array_equal(asum4, asum16)


# ----------------------------------------------------------------------------------
# MXFP8 (E4M3 elements, E8M0 scale per 32)
# ----------------------------------------------------------------------------------

E4M3_GRID = np.array(sorted(set(e4m3_decode_torch(np.arange(0x7F)).astype(np.float64))))


def test_mxfp8_storage_is_8p25_bits(orc):
    g = load("format_facts.json")
    R, Cc = 4, 64
    x = np.random.default_rng(1).standard_normal((R, Cc)).astype(np.float32)
    q = orc.quantize_mxfp8(x, 1, R, Cc)
    assert 8.0 * (q["codes"].nbytes + q["scales"].nbytes) / (R * Cc) == g["bits_per_value_mxfp8"]


def test_mxfp8_shared_exponent_closed_form(orc):
    # block maxima 1, 0.75, 448, 500, 2^-20: shared exponents -8, -9, 0, 0, -28
    x = np.zeros((5, 32), np.float32)
    for r, m in enumerate([1.0, 0.75, 448.0, 500.0, 2.0 ** -20]):
        x[r, 0] = m
        x[r, 1] = -m / 3
    q = orc.quantize_mxfp8(x, 1, 5, 32)
    assert list(q["scales"]) == [127 - 8, 127 - 9, 127, 127, 127 - 28]
    c = q["codes"].reshape(5, 32)
    assert c[2, 0] == 0x7E and c[3, 0] == 0x7E  # 448 exact; 500 saturates to 448
    assert orc.e8m0_value(q["scales"][0]) == 2.0 ** -8
    z = orc.quantize_mxfp8(np.zeros((1, 32), np.float32), 1, 1, 32)
    assert z["scales"][0] == 0 and (z["codes"] == 0).all()


def test_mxfp8_elements_match_torch_e4m3_cast(orc):
    """Below saturation every element is torch's RNE float8_e4m3fn cast of the value
    divided by its block's power-of-two scale (signed byte, zero as +0)."""
    rng = np.random.default_rng(5)
    R, Cc = 64, 256
    x = (rng.standard_normal((R, Cc)) * np.exp2(rng.uniform(-12, 12, (R, 1)))).astype(np.float32)
    q = orc.quantize_mxfp8(x, 1, R, Cc)
    scale = np.repeat(np.array([orc.e8m0_value(b) for b in q["scales"]]).reshape(R, Cc // 32), 32, 1)
    y = (x / scale).astype(np.float32)
    ok = np.abs(y) < 448.0
    ref = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ref = np.where((ref & 0x7F) == 0, 0, ref)  # -0 -> +0
    assert np.array_equal(q["codes"].reshape(R, Cc)[ok], ref[ok])
    assert ok.mean() > 0.99


def test_e4m3_sr_bracket_and_bias(orc):
    """E4M3 stochastic rounding: on-grid values are kept, others go to the lower or
    upper neighbour on torch's E4M3 grid, and over all 256 random bytes the mean is
    lo + (hi - lo) * ceil(256 p) / 256 with p = (a - lo)/(hi - lo): exactly unbiased
    when 256 p is an integer."""
    rng = np.random.default_rng(9)
    a_vals = np.concatenate([E4M3_GRID[:-1] + (E4M3_GRID[1:] - E4M3_GRID[:-1]) * rng.random(126),
                             E4M3_GRID[:-1] + (E4M3_GRID[1:] - E4M3_GRID[:-1]) * 0.25,
                             E4M3_GRID]).astype(np.float32)
    for a in a_vals:
        a64 = float(a)
        i = np.searchsorted(E4M3_GRID, a64, side="right") - 1
        lo = E4M3_GRID[i]
        codes = [orc.e4m3_sr(a, k) for k in range(256)]
        vals = np.array([orc.e4m3_value(c) for c in codes])
        if lo == a64 or a64 >= 448.0:
            assert (vals == min(a64, 448.0)).all()
            continue
        hi = E4M3_GRID[i + 1]
        assert set(vals) <= {lo, hi}
        p256 = Fraction(a64 - lo) / Fraction(hi - lo) * 256
        n_up = -(-p256.numerator // p256.denominator)  # ceil
        assert int((vals == hi).sum()) == n_up
    assert orc.e4m3_sr(500.0, 0) == 0x7E


def test_mxfp8_sr_transpose_is_exact_on_representable_values(orc):
    """NVFP4 values whose block scales are powers of two have at most 2 significant
    bits, so after the power-of-two MX scaling they are E4M3 values: the stochastic
    requantize must return the exact transpose for every seed."""
    rng = np.random.default_rng(13)
    R, Cc = 64, 48
    codes = rng.integers(0, 256, R * Cc // 2, dtype=np.uint8)
    scales = rng.choice(np.uint8([0x30, 0x38, 0x40, 0x48, 0x28]), R * Cc // 16)  # 2^-1 .. 2^2, 2^-2
    ts = np.float32([0.7])
    u = orc.dequantize(codes, scales, np.ones(1, np.float32), 1, R, Cc).reshape(R, Cc)
    for seed in [0, 1, 2 ** 33 + 5]:
        o = orc.requant_transpose_mxfp8_sr(codes, scales, ts, 1, R, Cc, seed)
        assert o["tensor_scale"][0] == ts[0]
        sc = np.repeat(np.array([orc.e8m0_value(b) for b in o["scales"]]).reshape(Cc, R // 32), 32, 1)
        v = e4m3_decode_torch(o["codes"]).astype(np.float64).reshape(Cc, R) * sc
        assert np.array_equal(v, u.T.astype(np.float64))


def test_mxfp8_sr_transpose_unbiased_over_seeds(orc):
    rng = np.random.default_rng(17)
    R, Cc = 64, 32
    codes = rng.integers(0, 256, R * Cc // 2, dtype=np.uint8)
    scales = rng.integers(0x20, 0x50, R * Cc // 16, dtype=np.uint8)
    u = orc.dequantize(codes, scales, np.ones(1, np.float32), 1, R, Cc).reshape(R, Cc).T
    acc = np.zeros((Cc, R))
    for seed in range(64):
        o = orc.requant_transpose_mxfp8_sr(codes, scales, np.float32([1.0]), 1, R, Cc, seed)
        sc = np.repeat(np.array([orc.e8m0_value(b) for b in o["scales"]]).reshape(Cc, R // 32), 32, 1)
        acc += e4m3_decode_torch(o["codes"]).astype(np.float64).reshape(Cc, R) * sc
    rel = (acc / 64 - u).sum() / np.abs(u).sum()
    assert abs(rel) < 2e-3, rel


# ----------------------------------------------------------------------------------
# 16x16-tile scaling
# ----------------------------------------------------------------------------------

def test_tile16_transpose_invariance(orc):
    """A transpose keeps every value's 16x16 tile, so quantizing the transposed
    tensor equals transposing the quantized one, bit for bit."""
    rng = np.random.default_rng(41)
    R, Cc = 48, 80
    x = rng.standard_normal((R, Cc)).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 30
    q = orc.quantize_tile16(x, 1, R, Cc)
    t = orc.transpose_tile16(q["codes"], q["scales"], q["tensor_scale"], 1, R, Cc)
    qt = orc.quantize_tile16(np.ascontiguousarray(x.T), 1, Cc, R)
    assert np.array_equal(t["codes"], qt["codes"])
    assert np.array_equal(t["scales"], qt["scales"])
    assert np.array_equal(t["tensor_scale"], qt["tensor_scale"])
    # and the transpose is an involution
    tt = orc.transpose_tile16(t["codes"], t["scales"], t["tensor_scale"], 1, Cc, R)
    assert np.array_equal(tt["codes"], q["codes"]) and np.array_equal(tt["scales"], q["scales"])


def test_tile16_reduces_to_block16_when_every_block_holds_the_tile_max(orc):
    """If each row block of 16 inside a tile already contains the tile's largest
    magnitude, tile and block scales coincide and so do all codes (Q is pinned)."""
    rng = np.random.default_rng(43)
    R, Cc = 32, 64
    x = rng.uniform(-1, 1, (R, Cc)).astype(np.float32)
    for ti in range(R // 16):
        for tj in range(Cc // 16):
            m = np.float32(rng.uniform(1.5, 40.0))
            for u in range(16):
                x[16 * ti + u, 16 * tj + rng.integers(16)] = m if rng.random() < 0.5 else -m
    q16 = orc.quantize_tile16(x, 1, R, Cc)
    qb = orc.quantize(x, 1, R, Cc)
    assert np.array_equal(q16["codes"], qb["codes"])
    tile_scales = q16["scales"].reshape(R // 16, Cc // 16)
    assert np.array_equal(np.repeat(tile_scales, 16, axis=0), qb["scales"].reshape(R, Cc // 16))


def test_tile16_one_large_value_zeros_its_tile(orc):
    """[TML] forward/backward-mismatch paragraph: one large value zeros the rest of
    its tile.  Closed form: with 1000 among 255 ones, s_t = 1000/2688 and the tile
    scale is E4M3 448 (d = (1000/6)/s_t = 448), so a one scales to
    y = 1/(448 s_t) = 0.006 -> code 0 while 1000 -> 6 (code 7); per-16 blocks zero
    only the 15 ones that share the large value's row block."""
    x = np.ones((16, 16), np.float32)
    x[0, 0] = 1000.0
    q16 = orc.quantize_tile16(x, 1, 16, 16)
    codes = unpack(q16["codes"], 256)
    assert q16["scales"][0] == 0x7E
    assert codes[0] == 7 and (codes[1:] == 0).all()
    qb = orc.quantize(x, 1, 16, 16)
    cb = unpack(qb["codes"], 256)
    assert cb[0] == 7 and (cb[1:16] == 0).all() and (cb[16:] != 0).all()


# ----------------------------------------------------------------------------------
# Mismatch statistics
# ----------------------------------------------------------------------------------

def test_mismatch_counts_small(orc):
    a = [0, 1, 2, 5, 9, 7, 15, 3, 1, 9]
    b = [0, 2, 2, 3, 1, 7, 14, 11, 10, 0]
    # mismatches: (1,2) (5,3) (9,1) (15,14) (3,11) (1,10) (9,0).
    # One step apart on the signed grid: (1,2) (15,14) (9,0) [-0.5 next to 0];
    # (1,10) is 0.5 vs -1.0 (three steps) although the magnitudes are adjacent.
    out = orc.code_mismatch(pack(a), pack(b), 1, 10)
    assert out.tolist() == [[7, 3]]
    out2 = orc.code_mismatch(pack(a + a), pack(b + a), 2, 10)
    assert out2.tolist() == [[7, 3], [0, 0]]

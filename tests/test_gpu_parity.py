"""GPU parity: libtq (HIP, through the C ABI) against the CPU oracle on the same
seeded inputs.  Codes, scales, tensor scales, hints, stochastic-rounding outputs,
dequantized values and counters must match bit for bit; the grouped GEMM must
satisfy |gpu - ref| <= 1e-3 * sum_k |a*w| for every checked output.

Full-size workloads are checked on samples the oracle computes one by one
(whole expert tensors, sampled token rows, sampled GEMM rows); small cases are
checked element by element.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from fp4_quantization_precision_amd import inputs, ops

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def npu8(t):
    return t.detach().cpu().contiguous().numpy().reshape(-1)


def hints_np(t):
    return t.detach().cpu().numpy().view(np.uint32).reshape(-1)


def assert_q_equal(g: ops.NVFP4, o: dict, what=""):
    torch.cuda.synchronize()
    assert np.array_equal(npu8(g.tensor_amax), o["tensor_amax"]), f"{what}: tensor amax"
    assert np.array_equal(npu8(g.tensor_scale), o["tensor_scale"]), f"{what}: tensor scale"
    assert np.array_equal(npu8(g.scales), o["scales"]), f"{what}: scales"
    gc, oc = npu8(g.codes), o["codes"]
    if not np.array_equal(gc, oc):
        bad = np.nonzero(gc != oc)[0]
        raise AssertionError(f"{what}: {bad.size} code bytes differ, first at byte {bad[0]}: "
                             f"gpu {gc[bad[0]]:#04x} oracle {oc[bad[0]]:#04x}")


def test_native_library_is_loaded():
    from fp4_quantization_precision_amd import _lib
    _lib.lib()
    maps = open("/proc/self/maps").read()
    assert os.path.realpath(_lib.LIB_PATH) in maps


# ----------------------------------------------------------------------------------
# Tiny NVFP4 round trip: 64x256 fp32
# ----------------------------------------------------------------------------------

def test_tiny_roundtrip_chain():
    xr, xt = inputs.tiny_roundtrip()
    n = xr.numel()
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV)
    qr = ops.quantize(xr.to(DEV), hints_out=hints)
    qn = ops.quantize(xt.to(DEV))
    qg = ops.quantize_guided(xt.to(DEV), hints)
    h2 = ops.extract_hint(qr.codes, n)
    cnt = ops.code_mismatch(torch.cat([qr.codes.reshape(-1)] * 2), torch.cat(
        [qn.codes.reshape(-1), qg.codes.reshape(-1)]), 2, n)
    o_r = oracle.quantize(xr, 1, 64, 256)
    o_n = oracle.quantize(xt, 1, 64, 256)
    o_h = oracle.extract_hint(o_r["codes"], n)
    o_g = oracle.quantize_guided(xt, 1, 64, 256, o_h)
    assert_q_equal(qr, o_r, "rollout")
    assert_q_equal(qn, o_n, "trainer nearest")
    assert_q_equal(qg, o_g, "trainer guided")
    assert np.array_equal(hints_np(hints), o_h)
    assert np.array_equal(hints_np(h2), o_h)
    o_c = oracle.code_mismatch(np.concatenate([o_r["codes"]] * 2),
                               np.concatenate([o_n["codes"], o_g["codes"]]), 2, n)
    got = cnt.cpu().numpy().astype(np.uint64)
    assert np.array_equal(got, o_c)
    assert got[1, 0] <= got[0, 0]
    print(f"\ntiny round trip: mismatches nearest {got[0, 0]} -> guided {got[1, 0]} of {n}")


# ----------------------------------------------------------------------------------
# Quantizer edge cases
# ----------------------------------------------------------------------------------

def _edge_tensor(kind, seed=0):
    rng = np.random.default_rng(seed)
    if kind == "all_zero":
        return np.zeros((2, 16, 64), np.float32)
    if kind == "neg_zero":
        x = rng.standard_normal((1, 8, 64)).astype(np.float32)
        x[0, :4] = -0.0
        return x
    if kind == "zero_and_subnormal_blocks":
        x = rng.standard_normal((3, 32, 96)).astype(np.float32)
        x[:, :, :16] = 0
        x[:, 3, 16:48] *= 2.0 ** -13
        x[:, 5, 48:64] *= 2.0 ** -17
        x[1, 0, 95] = 3000.0
        return x
    if kind == "midpoints":
        # unit scale (A_T = 2688, block max 6): every E2M1 midpoint and its neighbours
        mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
        vals = []
        for m in mids + [0.5, 1, 1.5, 2, 3, 4, 6, 6.5, 7.9]:
            v = np.float32(m)
            vals += [v, np.nextafter(v, np.float32(0)), np.nextafter(v, np.float32(10)), -v]
        per = 15
        nb = -(-len(vals) // per)
        x = np.zeros((1, 1, 16 * (nb + 1)), np.float32)
        for i, v in enumerate(vals):
            b, j = divmod(i, per)
            x[0, 0, 16 * b] = 6.0
            x[0, 0, 16 * b + 1 + j] = v
        x[0, 0, 16 * nb] = 2688.0
        return x
    if kind == "scale_rounds_down":
        # block max / 6 / s_t just below an E4M3 rounding tie: |y| exceeds 6 slightly
        x = rng.standard_normal((1, 64, 64)).astype(np.float32) * 0.1
        x[0, 0, 0] = 2688.0
        for r in range(1, 64):
            x[0, r, 0] = np.float32(6 * (1 + 1 / 16 - 1e-4) * (2.0 ** (r % 7)))
        return x
    if kind == "huge_and_tiny":
        x = rng.standard_normal((2, 16, 32)).astype(np.float32)
        x[0] *= 1e30
        x[1] *= 1e-28
        return x
    if kind == "single_row":
        return rng.standard_normal((1, 1, 16)).astype(np.float32)
    if kind == "many_small_tensors":
        return rng.standard_normal((300, 2, 32)).astype(np.float32) * rng.uniform(
            0.01, 100, (300, 1, 1)).astype(np.float32)
    if kind == "odd_block_count":
        return rng.standard_normal((1, 3, 16)).astype(np.float32)
    raise KeyError(kind)


EDGE = ["all_zero", "neg_zero", "zero_and_subnormal_blocks", "midpoints", "scale_rounds_down",
        "huge_and_tiny", "single_row", "many_small_tensors", "odd_block_count"]


@pytest.mark.parametrize("kind", EDGE)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_edges(kind, dtype):
    x = torch.from_numpy(_edge_tensor(kind))
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    B, R, Cc = x.shape
    n = x.numel()
    hints = torch.full((ops.hint_words(n),), -1, dtype=torch.int32, device=DEV)
    g = ops.quantize(x.to(DEV), hints_out=hints)
    o = oracle.quantize(x, B, R, Cc)
    assert_q_equal(g, o, kind)
    assert np.array_equal(hints_np(hints), oracle.extract_hint(o["codes"], n))
    # guided with a random hint stream
    rng = np.random.default_rng(1)
    h = rng.integers(0, 2 ** 32, ops.hint_words(n), dtype=np.uint64).astype(np.uint32)
    gg = ops.quantize_guided(x.to(DEV), torch.from_numpy(h.view(np.int32)).to(DEV))
    og = oracle.quantize_guided(x, B, R, Cc, h)
    assert_q_equal(gg, og, kind + " guided")
    # dequantization
    dq = ops.dequantize(g, B, R, Cc)
    torch.cuda.synchronize()
    assert np.array_equal(dq.cpu().numpy().reshape(-1).view(np.uint32),
                          oracle.dequantize(o["codes"], o["scales"], o["tensor_scale"], B, R,
                                            Cc).view(np.uint32))


@pytest.mark.parametrize("rows,cols,dtype", [
    (1, 16, "f32"), (3, 48, "bf16"), (517, 96, "bf16"), (300, 80, "f32"),
    (2048, 16384, "bf16"), (2049, 16400, "bf16"),
])
def test_quantize_from_scratch(rows, cols, dtype):
    """tq_quantize / tq_quantize_guided of one tensor without a given amax (amax pass,
    then quantize pass).  Bit-exact against the oracle for nearest, hints and guided,
    tensor amax and tensor scale included, on every element for small tensors and on
    sampled rows for the large ones."""
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_t(4, (rows, cols)) * 0.5).astype(np.float32)
    x[rng.random(x.shape) < 1e-3] *= 40
    xt = (x * (1 + rng.uniform(-2 ** -8, 2 ** -8, x.shape))).astype(np.float32)
    if dtype == "bf16":
        gx, gt = torch.from_numpy(x).to(torch.bfloat16), torch.from_numpy(xt).to(torch.bfloat16)
    else:
        gx, gt = torch.from_numpy(x), torch.from_numpy(xt)
    n = rows * cols
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV)
    qr = ops.quantize(gx.to(DEV), hints_out=hints)
    qg = ops.quantize_guided(gt.to(DEV), hints)
    qn = ops.quantize(gt.to(DEV))
    torch.cuda.synchronize()
    o_am_r = oracle.tensor_amax(gx, 1, n)
    o_am_t = oracle.tensor_amax(gt, 1, n)
    assert npu8(qr.tensor_amax)[0] == o_am_r[0] and npu8(qg.tensor_amax)[0] == o_am_t[0]
    sel = np.arange(rows) if rows <= 600 else np.unique(np.r_[0, rows - 1, rng.choice(rows, 40)])
    xs, ts_ = gx[sel].contiguous(), gt[sel].contiguous()
    R = sel.size
    o_r = oracle.quantize(xs, 1, R, cols, amax=o_am_r)
    o_n = oracle.quantize(ts_, 1, R, cols, amax=o_am_t)
    codes = lambda q: npu8(q.codes).reshape(rows, cols // 2)[sel].reshape(-1)
    scl = lambda q: npu8(q.scales).reshape(rows, cols // 16)[sel].reshape(-1)
    assert np.array_equal(codes(qr), o_r["codes"]) and np.array_equal(scl(qr), o_r["scales"])
    assert npu8(qr.tensor_scale)[0] == o_r["tensor_scale"][0]
    assert np.array_equal(codes(qn), o_n["codes"]) and np.array_equal(scl(qn), o_n["scales"])
    # hints of the sampled rows, then guided codes from them
    hw = hints_np(hints)
    o_h = oracle.extract_hint(o_r["codes"], R * cols)
    bits = np.unpackbits(hw.view(np.uint8), bitorder="little")[:n].reshape(rows, cols)[sel].reshape(-1)
    assert np.array_equal(np.unpackbits(o_h.view(np.uint8), bitorder="little")[:R * cols], bits)
    o_g = oracle.quantize_guided(ts_, 1, R, cols, o_h, amax=o_am_t)
    assert np.array_equal(codes(qg), o_g["codes"]) and np.array_equal(scl(qg), o_g["scales"])
    assert npu8(qg.tensor_scale)[0] == o_g["tensor_scale"][0]
    if rows <= 600:  # every element, and nothing written past the last hint word
        assert np.array_equal(hw[:ops.hint_words(n)], oracle.extract_hint(o_r["codes"], n))


@pytest.mark.parametrize("batch,n,dtype", [
    (1, 16, "bf16"), (1, 8 * 2 ** 20 + 48, "bf16"), (3, 4112, "f32"), (255, 1024, "bf16"),
    (256, 48, "bf16"), (300, 2064, "f32"),
])
def test_tensor_amax_batches(batch, n, dtype):
    """tq_tensor_amax over batches on both sides of the switch between the two launch
    shapes (1024-thread workgroups below 256 tensors, 256-thread workgroups from 256
    on), with the maximum at a random place per tensor, some tensors all zero and some
    holding subnormals only; bit-exact against the oracle."""
    rng = np.random.default_rng(batch * 131 + n)
    x = rng.standard_normal((batch, n)).astype(np.float32)
    where = rng.integers(0, n, batch)
    x[np.arange(batch), where] = rng.choice([-1, 1], batch) * rng.uniform(3, 300, batch)
    x[rng.random(batch) < 0.1] = 0.0
    sub = rng.random(batch) < 0.05
    x[sub] = np.float32(1e-40) * rng.standard_normal((int(sub.sum()), n)).astype(np.float32)
    g = torch.from_numpy(x).to(torch.bfloat16) if dtype == "bf16" else torch.from_numpy(x)
    am = ops.tensor_amax(g.to(DEV), batch=batch)
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), oracle.tensor_amax(g, batch, n))


def test_amax_given_and_tensor_amax():
    x = torch.from_numpy(_edge_tensor("zero_and_subnormal_blocks")).to(torch.bfloat16)
    B, R, Cc = x.shape
    am = ops.tensor_amax(x.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(am.cpu().numpy(), oracle.tensor_amax(x, B, R * Cc))
    out = ops.new_nvfp4((B,), R, Cc, DEV)
    out.tensor_amax.copy_(am)
    g = ops.quantize(x.to(DEV), out=out, amax_given=True)
    assert_q_equal(g, oracle.quantize(x, B, R, Cc), "amax given")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_more_tensors_than_grid_rows(dtype):
    """65541 tensors of 2 x 16 values: more tensors than the launch has workgroup rows
    (65535), so the quantizers and the mismatch count take their looping path over
    tensors.  Nearest with hints, guided, from-scratch amax and the per-tensor
    mismatch counts, bit-exact against the oracle on every tensor."""
    B, R, Cc = 65541, 2, 16
    rng = np.random.default_rng(65541)
    x = (rng.standard_normal((B, R, Cc)) * np.exp2(rng.integers(-20, 20, (B, 1, 1)))).astype(np.float32)
    x[rng.random(B) < 0.01] = 0.0
    xt = (x * (1 + rng.uniform(-2 ** -8, 2 ** -8, x.shape))).astype(np.float32)
    if dtype == "bf16":
        gx, gt = torch.from_numpy(x).to(torch.bfloat16), torch.from_numpy(xt).to(torch.bfloat16)
    else:
        gx, gt = torch.from_numpy(x), torch.from_numpy(xt)
    n = B * R * Cc
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV)
    qr = ops.quantize(gx.to(DEV), hints_out=hints)
    qg = ops.quantize_guided(gt.to(DEV), hints)
    torch.cuda.synchronize()
    o_r = oracle.quantize(gx, B, R, Cc)
    assert_q_equal(qr, o_r, "rollout")
    o_h = oracle.extract_hint(o_r["codes"], n)
    assert np.array_equal(hints_np(hints), o_h)
    o_g = oracle.quantize_guided(gt, B, R, Cc, o_h)
    assert_q_equal(qg, o_g, "guided")
    # guided codes match the rollout's here, so count against the trainer's nearest codes
    qn = ops.quantize(gt.to(DEV))
    cnt = ops.code_mismatch(qr.codes.reshape(-1), qn.codes.reshape(-1), B, R * Cc)
    torch.cuda.synchronize()
    o_n = oracle.quantize(gt, B, R, Cc)
    assert_q_equal(qn, o_n, "trainer nearest")
    want = oracle.code_mismatch(o_r["codes"].reshape(-1), o_n["codes"].reshape(-1), B, R * Cc)
    assert want[:, 0].sum() > 0
    assert np.array_equal(cnt.cpu().numpy().astype(np.uint64), want)


def test_empty_tensors():
    x = torch.zeros((3, 0, 32), dtype=torch.bfloat16, device=DEV)
    out = ops.new_nvfp4((3,), 0, 32, DEV)
    out.tensor_scale.fill_(7.0)
    out.tensor_amax.fill_(7.0)
    ops.quantize(x, out=out)
    torch.cuda.synchronize()
    assert (out.tensor_scale == 0).all() and (out.tensor_amax == 0).all()
    q = ops.NVFP4(torch.zeros(0, dtype=torch.uint8, device=DEV),
                  torch.zeros(0, dtype=torch.uint8, device=DEV),
                  torch.tensor([0.5, 2.0], device=DEV), torch.zeros(2, device=DEV))
    t = ops.requant_transpose_sr(q, 2, 0, 32, seed=1)
    torch.cuda.synchronize()
    assert t.tensor_scale.cpu().tolist() == [0.5, 2.0]


def test_boundary_example_from_trace_page():
    g = json.load(open(os.path.join(GOLDEN, "rounding_boundary.json")))
    xr = np.zeros((1, 1, 32), np.float32)
    xt = np.zeros((1, 1, 32), np.float32)
    xr[0, 0, 0] = xt[0, 0, 0] = 6.0
    xr[0, 0, 16] = xt[0, 0, 16] = 2688.0
    xr[0, 0, 1], xt[0, 0, 1] = g["rollout_value"], g["train_value"]
    h = torch.zeros(1, dtype=torch.int32, device=DEV)
    qr = ops.quantize(torch.from_numpy(xr).to(DEV), hints_out=h)
    qn = ops.quantize(torch.from_numpy(xt).to(DEV))
    qg = ops.quantize_guided(torch.from_numpy(xt).to(DEV), h)
    torch.cuda.synchronize()
    code = lambda q: int(q.codes.cpu()[0, 0, 0] >> 4)
    assert code(qr) == g["rollout_nearest_code"]
    assert code(qn) == g["train_nearest_code"]
    assert code(qg) == g["train_guided_code"]


# ----------------------------------------------------------------------------------
# Hints
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 64, 1000, 4112, 1 << 20, (1 << 20) + 46])
def test_extract_hint(n):
    rng = np.random.default_rng(n)
    codes = rng.integers(0, 256, (n + 1) // 2 + 16, dtype=np.uint8)
    words = ops.hint_words(n)
    h = torch.full((words + 2,), -1, dtype=torch.int32, device=DEV)
    ops.extract_hint(torch.from_numpy(codes).to(DEV), n, h)
    torch.cuda.synchronize()
    got = hints_np(h)
    assert np.array_equal(got[:words], oracle.extract_hint(codes, n))
    assert (got[words:] == 0xFFFFFFFF).all()  # nothing written past the hint words


# ----------------------------------------------------------------------------------
# MoE expert weights: 48 layers x 64 experts x [2048 x 768] bf16 (two full layers)
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("layer", [0, 24, 47])
def test_moe_weights_layer_full_size(layer):
    E, R, Cc, L = 64, 2048, 768, 48
    xr, xt = inputs.moe_expert_weights_layer(layer, E, R, Cc, device=DEV)
    n = xr.numel()
    with_hints = layer >= ops.hint_first_layer(L)
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV) if with_hints else None
    qr = ops.quantize(xr, hints_out=hints)
    qn = ops.quantize(xt)
    qg = ops.quantize_guided(xt, hints, out=ops.new_nvfp4((E,), R, Cc, DEV)) if with_hints else qn
    before = ops.code_mismatch(qr.codes.reshape(-1), qn.codes.reshape(-1), E, R * Cc)
    after = ops.code_mismatch(qr.codes.reshape(-1), qg.codes.reshape(-1), E, R * Cc)
    torch.cuda.synchronize()
    per = R * Cc
    # the hinted layer 24 is compared on every expert, the others on three
    experts = range(E) if layer == 24 else [0, 17, E - 1]
    xr_h, xt_h = xr.cpu(), xt.cpu()
    qr_c, qr_s, qn_c = npu8(qr.codes), npu8(qr.scales), npu8(qn.codes)
    qg_c, qg_s, qr_t = npu8(qg.codes), npu8(qg.scales), npu8(qr.tensor_scale)
    h_np = hints_np(hints) if with_hints else None
    bef, aft = before.cpu().numpy(), after.cpu().numpy()

    def check_expert(e):
        xr_e, xt_e = xr_h[e], xt_h[e]
        o_r = oracle.quantize(xr_e, 1, R, Cc)
        o_n = oracle.quantize(xt_e, 1, R, Cc)
        sl = lambda a, div: a[e * per // div:(e + 1) * per // div]
        assert np.array_equal(sl(qr_c, 2), o_r["codes"]), f"expert {e} rollout codes"
        assert np.array_equal(sl(qr_s, 16), o_r["scales"]), f"expert {e} rollout scales"
        assert qr_t[e] == o_r["tensor_scale"][0]
        assert np.array_equal(sl(qn_c, 2), o_n["codes"]), f"expert {e} trainer codes"
        o_cn = oracle.code_mismatch(o_r["codes"], o_n["codes"], 1, per)
        assert np.array_equal(bef[e].astype(np.uint64), o_cn[0])
        if with_hints:
            o_h = oracle.extract_hint(o_r["codes"], per)
            assert np.array_equal(h_np[e * per // 32:(e + 1) * per // 32], o_h)
            o_g = oracle.quantize_guided(xt_e, 1, R, Cc, o_h)
            assert np.array_equal(sl(qg_c, 2), o_g["codes"]), f"expert {e} guided codes"
            assert np.array_equal(sl(qg_s, 16), o_g["scales"])
            o_cg = oracle.code_mismatch(o_r["codes"], o_g["codes"], 1, per)
            assert np.array_equal(aft[e].astype(np.uint64), o_cg[0])

    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=8) as ex:
        list(ex.map(check_expert, experts))
    b, a = before.sum(0).tolist(), after.sum(0).tolist()
    assert a[0] <= b[0]
    print(f"\nlayer {layer}: mismatch rate nearest {b[0] / n:.3e} (adjacent {b[1] / max(b[0], 1):.4f})"
          f" -> {'guided' if with_hints else 'nearest'} {a[0] / n:.3e}")


def test_moe_step_launches():
    """The step's streaming launches at full size: 48 layers x 64 experts of
    [2048 x 768] bf16 in one call each (3072 tensors, 4.8e9 values, so flattened
    indices pass 2^32), as the benchmark issues them: tensor amax of both copies,
    nearest quantize of the rollout copy (layers 0-23) and nearest + hints (layers
    24-47, 1536 tensors), nearest of the trainer copy over all 48 layers, guided
    over layers 24-47 with those hints, and both mismatch counts.  Sampled tensors
    (first, middle and last of each launch) are bit-exact against the oracle,
    computed on that tensor alone."""
    L, E, R, Cc = 48, 64, 2048, 768
    fh = ops.hint_first_layer(L)
    XR = torch.empty((L, E, R, Cc), dtype=torch.bfloat16, device=DEV)
    XT = torch.empty_like(XR)
    for layer in range(L):
        XR[layer], XT[layer] = inputs.moe_expert_weights_layer(layer, E, R, Cc, device=DEV)
    per = R * Cc
    n_h = (L - fh) * E * per
    QR = ops.new_nvfp4((L, E), R, Cc, DEV)
    QN = ops.new_nvfp4((L, E), R, Cc, DEV)
    QG = ops.new_nvfp4((L - fh, E), R, Cc, DEV)
    H = torch.zeros(ops.hint_words(n_h), dtype=torch.int32, device=DEV)
    ops.tensor_amax(XR, QR.tensor_amax, batch=L * E)
    # layers [a, b) of a batch: codes and scales are [L][E][...], the scalars flat [L * E]
    sub = lambda q, a, b: ops.NVFP4(q.codes[a:b], q.scales[a:b], q.tensor_scale[a * E:b * E],
                                    q.tensor_amax[a * E:b * E])
    ops.quantize(XR[:fh], out=sub(QR, 0, fh), amax_given=True)
    ops.quantize(XR[fh:], out=sub(QR, fh, L), hints_out=H, amax_given=True)
    ops.tensor_amax(XT, QN.tensor_amax, batch=L * E)
    ops.quantize(XT, out=QN, amax_given=True)
    QG.tensor_amax.copy_(QN.tensor_amax[fh * E:])
    ops.quantize_guided(XT[fh:], H, out=QG, amax_given=True)
    cnt_n = ops.code_mismatch(QR.codes.reshape(-1), QN.codes.reshape(-1), L * E, per)
    cnt_g = ops.code_mismatch(QR.codes[fh:].reshape(-1), QG.codes.reshape(-1), (L - fh) * E, per)
    torch.cuda.synchronize()
    flat = lambda t: t.reshape(-1)
    ar_all, an_all = QR.tensor_amax.reshape(-1).cpu(), QN.tensor_amax.reshape(-1).cpu()
    for t in [0, 1537, L * E - 1]:  # one 3072-tensor launch index each
        layer, e = divmod(t, E)
        xr, xt = XR[layer, e].cpu(), XT[layer, e].cpu()
        assert ar_all[t].item() == xr.float().abs().max().item(), f"rollout amax {t}"
        assert an_all[t].item() == xt.float().abs().max().item(), f"trainer amax {t}"
        o_r = oracle.quantize(xr, 1, R, Cc)
        o_n = oracle.quantize(xt, 1, R, Cc)
        assert np.array_equal(npu8(flat(QR.codes[layer, e])), o_r["codes"]), f"rollout codes {t}"
        assert np.array_equal(npu8(flat(QR.scales[layer, e])), o_r["scales"]), f"rollout scales {t}"
        assert np.array_equal(npu8(flat(QN.codes[layer, e])), o_n["codes"]), f"trainer codes {t}"
        assert np.array_equal(npu8(flat(QN.scales[layer, e])), o_n["scales"]), f"trainer scales {t}"
        assert np.array_equal(npu8(QN.tensor_scale[t:t + 1]), o_n["tensor_scale"])
        o_c = oracle.code_mismatch(o_r["codes"], o_n["codes"], 1, per)
        assert np.array_equal(cnt_n[t].cpu().numpy().astype(np.uint64), o_c[0]), f"mismatch {t}"
    h_all = hints_np(H)
    for tr in [0, 777, (L - fh) * E - 1]:  # index in the 1536-tensor launches
        t = fh * E + tr
        layer, e = divmod(t, E)
        xr, xt = XR[layer, e].cpu(), XT[layer, e].cpu()
        o_r = oracle.quantize(xr, 1, R, Cc)
        o_h = oracle.extract_hint(o_r["codes"], per)
        assert np.array_equal(h_all[tr * per // 32:(tr + 1) * per // 32], o_h), f"hints {tr}"
        o_g = oracle.quantize_guided(xt, 1, R, Cc, o_h)
        ql, qe = divmod(tr, E)
        assert np.array_equal(npu8(flat(QG.codes[ql, qe])), o_g["codes"]), f"guided codes {tr}"
        assert np.array_equal(npu8(flat(QG.scales[ql, qe])), o_g["scales"]), f"guided scales {tr}"
        o_c = oracle.code_mismatch(o_r["codes"], o_g["codes"], 1, per)
        assert np.array_equal(cnt_g[tr].cpu().numpy().astype(np.uint64), o_c[0]), f"guided mismatch {tr}"


# ----------------------------------------------------------------------------------
# Activations: 32768 x 4096 bf16, Student-t(4) with 8 outlier channels
# ----------------------------------------------------------------------------------

def test_activations_full_size():
    T, H = 32768, 4096
    xr, xt, _ = inputs.activations(T, H, device=DEV)
    n = xr.numel()
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV)
    qr = ops.quantize(xr, hints_out=hints)
    qg = ops.quantize_guided(xt, hints)
    qn = ops.quantize(xt)
    cnt = ops.code_mismatch(torch.cat([qr.codes.reshape(-1)] * 2),
                            torch.cat([qn.codes.reshape(-1), qg.codes.reshape(-1)]), 2, n)
    torch.cuda.synchronize()
    xr_c, xt_c = xr.cpu(), xt.cpu()
    am_r = oracle.tensor_amax(xr_c, 1, n)
    am_t = oracle.tensor_amax(xt_c, 1, n)
    assert npu8(qr.tensor_amax)[0] == am_r[0] and npu8(qg.tensor_amax)[0] == am_t[0]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 61, replace=False)]))
    for r in rows:
        o_r = oracle.quantize(xr_c[r:r + 1], 1, 1, H, amax=am_r)
        o_h = oracle.extract_hint(o_r["codes"], H)
        o_g = oracle.quantize_guided(xt_c[r:r + 1], 1, 1, H, o_h, amax=am_t)
        assert np.array_equal(npu8(qr.codes[r]), o_r["codes"]), f"row {r}"
        assert np.array_equal(npu8(qr.scales[r]), o_r["scales"]), f"row {r}"
        assert np.array_equal(hints_np(hints)[r * H // 32:(r + 1) * H // 32], o_h), f"row {r}"
        assert np.array_equal(npu8(qg.codes[r]), o_g["codes"]), f"row {r} guided"
        assert np.array_equal(npu8(qg.scales[r]), o_g["scales"]), f"row {r} guided"
    c = cnt.cpu().numpy()
    assert c[1, 0] <= c[0, 0]
    print(f"\nactivations: mismatch rate nearest {c[0, 0] / n:.3e} -> guided {c[1, 0] / n:.3e}")


@pytest.mark.parametrize("which", ["K", "V"])
def test_kv_cache_full_size(which):
    """FP4 KV cache with hints: one layer's K (or V) cache [32768 x 8 x 128] quantized
    per token-head (blocks of 16 along head_dim, one tensor scale), rollout nearest +
    hints, trainer guided; sampled token-heads bit-exact against the oracle, full
    mismatch counts checked against the oracle's on the same rows."""
    T, Hh, D = 32768, 8, 128
    kr, kt, vr, vt, _ = inputs.kv_cache(T, Hh, D, device=DEV)
    xr, xt = (kr, kt) if which == "K" else (vr, vt)
    R = T * Hh
    n = xr.numel()
    hints = torch.zeros(ops.hint_words(n), dtype=torch.int32, device=DEV)
    qr = ops.quantize(xr.view(1, R, D), hints_out=hints)
    qg = ops.quantize_guided(xt.view(1, R, D), hints)
    qn = ops.quantize(xt.view(1, R, D))
    cnt = ops.code_mismatch(torch.cat([qr.codes.reshape(-1)] * 2),
                            torch.cat([qn.codes.reshape(-1), qg.codes.reshape(-1)]), 2, n)
    torch.cuda.synchronize()
    xr_c, xt_c = xr.reshape(R, D).cpu(), xt.reshape(R, D).cpu()
    am_r = oracle.tensor_amax(xr_c, 1, n)
    am_t = oracle.tensor_amax(xt_c, 1, n)
    assert npu8(qr.tensor_amax)[0] == am_r[0] and npu8(qg.tensor_amax)[0] == am_t[0]
    rng = np.random.default_rng(1)
    rows = np.unique(np.concatenate([[0, 1, R - 1], rng.choice(R, 509, replace=False)]))
    o_r = oracle.quantize(xr_c[rows], 1, rows.size, D, amax=am_r)
    o_h = oracle.extract_hint(o_r["codes"], rows.size * D)
    o_g = oracle.quantize_guided(xt_c[rows], 1, rows.size, D, o_h, amax=am_t)
    o_n = oracle.quantize(xt_c[rows], 1, rows.size, D, amax=am_t)
    codes_r = npu8(qr.codes).reshape(R, D // 2)[rows].reshape(-1)
    codes_g = npu8(qg.codes).reshape(R, D // 2)[rows].reshape(-1)
    codes_n = npu8(qn.codes).reshape(R, D // 2)[rows].reshape(-1)
    assert np.array_equal(codes_r, o_r["codes"])
    assert np.array_equal(npu8(qr.scales).reshape(R, D // 16)[rows].reshape(-1), o_r["scales"])
    assert np.array_equal(hints_np(hints).reshape(R, D // 32)[rows].reshape(-1), o_h)
    assert np.array_equal(codes_g, o_g["codes"])
    assert np.array_equal(npu8(qg.scales).reshape(R, D // 16)[rows].reshape(-1), o_g["scales"])
    assert np.array_equal(codes_n, o_n["codes"])
    c = cnt.cpu().numpy()
    assert c[1, 0] <= c[0, 0]
    print(f"\nKV cache {which}: mismatch rate nearest {c[0, 0] / n:.3e} "
          f"(adjacent {c[0, 1] / max(c[0, 0], 1):.3f}) -> guided {c[1, 0] / n:.3e}")


# ----------------------------------------------------------------------------------
# MXFP8 for the backward
# ----------------------------------------------------------------------------------

MX_SHAPES = [(1, 1, 32, "f32"), (1, 4, 64, "bf16"), (3, 17, 96, "bf16"), (2, 5, 1056, "f32"),
             (1, 257, 512, "bf16")]


@pytest.mark.parametrize("shape", MX_SHAPES)
def test_mxfp8_quantize_shapes(shape):
    B, R, Cc, dt = shape
    rng = np.random.default_rng(R * 31 + Cc)
    x = (rng.standard_normal((B, R, Cc)) * np.exp2(rng.uniform(-30, 30, (B, R, 1)))).astype(np.float32)
    x[rng.random(x.shape) < 0.01] *= 1000
    x.reshape(-1)[:32] = 0.0                     # an all-zero block
    x.reshape(-1)[32:64] *= 2.0 ** -120           # a block near the bottom of the range
    if x.size >= 96:
        # shared exponent 0: saturation at 448 from above, negative values that round to
        # zero (written +0), -0, ties to even in the normal and subnormal ranges, the
        # smallest subnormal (all exact in bf16 too)
        edge = [480.0, -464.0, 456.0, -2.0 ** -11, -2.0 ** -10, -3 * 2.0 ** -11, 0.0, -0.0,
                1.0625, 1.1875, -1.0625, 3 * 2.0 ** -10, -2.0 ** -9, 2.0 ** -7 + 2.0 ** -10, 448.0, -448.0]
        x.reshape(-1)[64:96] = np.float32(edge + edge[::-1])
    xt = torch.from_numpy(x)
    if dt == "bf16":
        xt = xt.to(torch.bfloat16)
    q = ops.quantize_mxfp8(xt.to(DEV))
    torch.cuda.synchronize()
    o = oracle.quantize_mxfp8(xt, B, R, Cc)
    assert np.array_equal(npu8(q.codes), o["codes"])
    assert np.array_equal(npu8(q.scales), o["scales"])


def test_mxfp8_quantize_activations_full_size():
    """The activations workload (32768 x 4096 bf16) at full size on the device;
    blocks are row-local, so 515 sampled rows (first, last and random) are checked
    bit-exact against the oracle run on those rows."""
    T, Hd = 32768, 4096
    xr, _, _ = inputs.activations(T, Hd, device=DEV)
    q = ops.quantize_mxfp8(xr)
    torch.cuda.synchronize()
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([[0, 1, T - 1], rng.choice(T, 512, replace=False)]))
    o = oracle.quantize_mxfp8(xr.cpu()[rows], 1, rows.size, Hd)
    assert np.array_equal(npu8(q.codes).reshape(T, Hd)[rows].reshape(-1), o["codes"])
    assert np.array_equal(npu8(q.scales).reshape(T, Hd // 32)[rows].reshape(-1), o["scales"])


MX_SR_SHAPES = [(1, 32, 16), (1, 64, 80), (3, 288, 96), (2, 32, 1040), (1, 1024, 1024)]


@pytest.mark.parametrize("shape", MX_SR_SHAPES)
def test_mxfp8_sr_transpose_shapes(shape):
    B, R, Cc = shape
    c, s, ts = inputs.random_nvfp4(B, R, Cc, seed=R + 3 * Cc, zero_block_frac=0.05)
    q = ops.NVFP4(c.to(DEV), s.to(DEV), ts.to(DEV), torch.zeros(B, device=DEV))
    for seed in [0, 2 ** 40 + 3]:
        t = ops.requant_transpose_mxfp8_sr(q, B, R, Cc, seed)
        torch.cuda.synchronize()
        o = oracle.requant_transpose_mxfp8_sr(c, s, ts, B, R, Cc, seed)
        assert np.array_equal(npu8(t.codes), o["codes"]), f"{shape} seed {seed}"
        assert np.array_equal(npu8(t.scales), o["scales"]), f"{shape} seed {seed}"
        assert np.array_equal(npu8(t.tensor_scale), o["tensor_scale"])


def test_mxfp8_sr_transpose_full_size():
    """The 8192^2 transpose source, nearest NVFP4, then the MXFP8 backward copy."""
    N = 8192
    x = inputs.transpose_source(N, N, device=DEV)
    q = ops.quantize(x)
    t = ops.requant_transpose_mxfp8_sr(q, 1, N, N, seed=11)
    torch.cuda.synchronize()
    o = oracle.quantize(x.cpu(), 1, N, N)
    assert_q_equal(q, o, "8192^2 nearest")
    ot = oracle.requant_transpose_mxfp8_sr(o["codes"], o["scales"], o["tensor_scale"], 1, N, N, 11)
    assert np.array_equal(npu8(t.codes), ot["codes"])
    assert np.array_equal(npu8(t.scales), ot["scales"])



def test_mxfp8_sr_transpose_moe_layer():
    """One MoE layer per call (64 experts of [2048 x 768], 3072 tiles), the launch the
    MXFP8 backward copy of the expert weights takes; sampled experts bit-exact against
    the oracle, recomputed alone with their index in the batch."""
    B, R, Cc = 64, 2048, 768
    c, s, ts = inputs.random_nvfp4(B, R, Cc, seed=31, device=DEV, zero_block_frac=0.02)
    q = ops.NVFP4(c, s, ts, torch.zeros(B, device=DEV))
    t = ops.requant_transpose_mxfp8_sr(q, B, R, Cc, seed=47)
    torch.cuda.synchronize()
    per = R * Cc
    for b in [0, 31, B - 1]:
        o = oracle.requant_transpose_mxfp8_sr(npu8(c[b]), npu8(s[b]), npu8(ts[b:b + 1]),
                                              1, R, Cc, 47, first=b)
        assert np.array_equal(npu8(t.codes.reshape(-1)[b * per:(b + 1) * per]), o["codes"]), f"expert {b}"
        assert np.array_equal(npu8(t.scales.reshape(-1)[b * per // 32:(b + 1) * per // 32]), o["scales"])


# ----------------------------------------------------------------------------------
# 16x16-tile scaling
# ----------------------------------------------------------------------------------

TILE16_SHAPES = [(1, 16, 16, "f32"), (1, 48, 80, "bf16"), (3, 272, 96, "bf16"), (2, 16, 1040, "f32"),
                 (1, 64, 64, "bf16"), (2, 528, 144, "bf16"), (1, 1024, 1024, "f32"),
                 (1, 592, 832, "bf16")]  # 481 wave units: a grid that is not a multiple of 8 workgroups


@pytest.mark.parametrize("shape", TILE16_SHAPES)
def test_tile16_shapes(shape):
    B, R, Cc, dt = shape
    rng = np.random.default_rng(R * 7 + Cc)
    x = rng.standard_normal((B, R, Cc)).astype(np.float32)
    x[rng.random(x.shape) < 0.003] *= 60
    x[:, :16, :16] = 0.0  # an all-zero tile
    xt = torch.from_numpy(x)
    if dt == "bf16":
        xt = xt.to(torch.bfloat16)
    q = ops.quantize_tile16(xt.to(DEV))
    t = ops.transpose_tile16(q, B, R, Cc)
    tq_ = ops.quantize_tile16(xt.transpose(-1, -2).contiguous().to(DEV))
    torch.cuda.synchronize()
    o = oracle.quantize_tile16(xt, B, R, Cc)
    ot = oracle.transpose_tile16(o["codes"], o["scales"], o["tensor_scale"], B, R, Cc)
    assert np.array_equal(npu8(q.codes), o["codes"])
    assert np.array_equal(npu8(q.scales), o["scales"])
    assert np.array_equal(npu8(q.tensor_scale), o["tensor_scale"])
    assert np.array_equal(npu8(t.codes), ot["codes"])
    assert np.array_equal(npu8(t.scales), ot["scales"])
    assert np.array_equal(npu8(t.tensor_scale), ot["tensor_scale"])
    # transpose invariance on the device
    assert np.array_equal(npu8(tq_.codes), npu8(t.codes))
    assert np.array_equal(npu8(tq_.scales), npu8(t.scales))


def test_tile16_activations_full_size():
    """The activations workload (32768 x 4096 bf16, 8 outlier channels x50) with
    16x16 tiles: codes, scales and the exact transpose bit-exact against the oracle;
    the fraction of nonzero values zeroed is reported against block-16 scaling."""
    T, Hd = 32768, 4096
    xr, _, _ = inputs.activations(T, Hd, device=DEV)
    q = ops.quantize_tile16(xr)
    t = ops.transpose_tile16(q, 1, T, Hd)
    qb = ops.quantize(xr)
    torch.cuda.synchronize()
    xc = xr.cpu()
    o = oracle.quantize_tile16(xc, 1, T, Hd)
    assert np.array_equal(npu8(q.codes), o["codes"])
    assert np.array_equal(npu8(q.scales), o["scales"])
    ot = oracle.transpose_tile16(o["codes"], o["scales"], o["tensor_scale"], 1, T, Hd)
    assert np.array_equal(npu8(t.codes), ot["codes"])
    assert np.array_equal(npu8(t.scales), ot["scales"])
    nz = (xc != 0).numpy().reshape(-1)
    c16 = oracle.unpack_codes(npu8(q.codes), T * Hd)
    cb = oracle.unpack_codes(npu8(qb.codes), T * Hd)
    z16 = float(((c16 & 7) == 0)[nz].mean())
    zb = float(((cb & 7) == 0)[nz].mean())
    assert z16 > zb
    print(f"\nactivations: nonzero values quantized to 0: 16x16 tiles {z16:.4f}, 1x16 blocks {zb:.4f}")


# ----------------------------------------------------------------------------------
# Transpose-requantize with stochastic rounding
# ----------------------------------------------------------------------------------

def test_transpose_sr_full_size():
    """The whole 8192^2 tensor, bit-exact for seeds 0, 1 and 63."""
    N = 8192
    x = inputs.transpose_source(N, N, device=DEV)
    q = ops.quantize(x)
    torch.cuda.synchronize()
    xc = x.cpu()
    o = oracle.quantize(xc, 1, N, N)
    assert_q_equal(q, o, "8192^2 nearest")
    for seed in (0, 1, 63):
        t = ops.requant_transpose_sr(q, 1, N, N, seed=seed)
        torch.cuda.synchronize()
        ot = oracle.requant_transpose_sr(o["codes"], o["scales"], o["tensor_scale"], 1, N, N, seed)
        assert np.array_equal(npu8(t.codes), ot["codes"]), f"seed {seed}"
        assert np.array_equal(npu8(t.scales), ot["scales"]), f"seed {seed}"
        assert np.array_equal(npu8(t.tensor_scale), ot["tensor_scale"]), f"seed {seed}"



def test_transpose_sr_moe_step_launch():
    """The MoE step's launch: 24 layers x 64 experts of [2048 x 768] in one call
    (73728 tiles; each workgroup walks nine).  Tensors 0, 777 and 1535 come from the
    first, a middle and the last tile of their workgroups' walks; bit-exact against
    the oracle, recomputed alone with their index in the batch, for both seeds the
    step uses."""
    B, R, Cc = 24 * 64, 2048, 768
    c, s, ts = inputs.random_nvfp4(B, R, Cc, seed=29, device=DEV, zero_block_frac=0.02)
    q = ops.NVFP4(c, s, ts, torch.zeros(B, device=DEV))
    per = R * Cc
    for seed in [0, 1]:
        t = ops.requant_transpose_sr(q, B, R, Cc, seed=seed)
        torch.cuda.synchronize()
        for b in [0, 777, B - 1]:
            o = oracle.requant_transpose_sr(npu8(c[b]), npu8(s[b]), npu8(ts[b:b + 1]),
                                            1, R, Cc, seed, first=b)
            got = npu8(t.codes.reshape(-1)[b * per // 2:(b + 1) * per // 2])
            assert np.array_equal(got, o["codes"]), f"seed {seed} tensor {b}"
            got = npu8(t.scales.reshape(-1)[b * per // 16:(b + 1) * per // 16])
            assert np.array_equal(got, o["scales"]), f"seed {seed} tensor {b}"
            assert npu8(t.tensor_scale[b:b + 1])[0] == o["tensor_scale"][0]


SR_SHAPES = [(1, 16, 16), (1, 48, 80), (3, 272, 96), (2, 16, 1040), (1, 32, 64), (2, 528, 144),
             (1, 256, 64), (1, 1024, 1024),
             # 900 tiles, ragged in both directions, on 512 workgroups: workgroups walk one or
             # two tiles, prefetching partial tiles after full ones and the reverse
             (100, 272, 528)]


@pytest.mark.parametrize("shape", SR_SHAPES)
def test_transpose_sr_shapes(shape):
    B, R, Cc = shape
    c, s, ts = inputs.random_nvfp4(B, R, Cc, seed=R + Cc, zero_block_frac=0.05)
    q = ops.NVFP4(c.to(DEV), s.to(DEV), ts.to(DEV), torch.zeros(B, device=DEV))
    for seed in [0, 2 ** 40 + 3]:
        t = ops.requant_transpose_sr(q, B, R, Cc, seed=seed)
        torch.cuda.synchronize()
        o = oracle.requant_transpose_sr(c, s, ts, B, R, Cc, seed)
        assert np.array_equal(npu8(t.codes), o["codes"]), f"{shape} seed {seed}"
        assert np.array_equal(npu8(t.scales), o["scales"]), f"{shape} seed {seed}"
        assert np.array_equal(npu8(t.tensor_scale), o["tensor_scale"])


def test_transpose_sr_on_grid_exact():
    """Every requantized value on the grid (one scale for the whole tensor and a 6
    in every new block): for every seed the transpose reproduces the input codes,
    with -0 written as +0 -- the step-up test must treat t == |y| as no step."""
    B, R, Cc = 1, 64, 96
    rng = np.random.default_rng(17)
    codes4 = rng.integers(0, 16, size=(R, Cc), dtype=np.uint8)
    codes4[::16, :] = np.where(rng.random(Cc) < 0.5, 7, 15).astype(np.uint8)  # +-6 in each new block
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    c = torch.from_numpy(packed)
    s = torch.full((R * Cc // 16,), 0x38, dtype=torch.uint8)  # every block scale 1.0
    ts = torch.ones(1, dtype=torch.float32)
    q = ops.NVFP4(c.to(DEV), s.to(DEV), ts.to(DEV), torch.zeros(B, device=DEV))
    want = codes4.T.copy()
    want[want == 8] = 0
    want_packed = (want[:, 0::2] | (want[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    for seed in range(4):
        t = ops.requant_transpose_sr(q, B, R, Cc, seed=seed)
        torch.cuda.synchronize()
        o = oracle.requant_transpose_sr(c, s, ts, B, R, Cc, seed)
        assert np.array_equal(npu8(t.codes), o["codes"]), f"seed {seed}"
        assert np.array_equal(npu8(t.codes), want_packed), f"seed {seed}"
        assert np.all(npu8(t.scales) == 0x38)


def test_transpose_sr_block_scale_rounds_to_zero():
    """New blocks whose largest value is nonzero but so small that A/6 rounds to the
    E4M3 code 0 (every input scale 2^-9 and every code of magnitude 0 or 0.5 in a band
    of 16 rows, so A <= 2^-10), next to all-zero new blocks (zero codes under a nonzero
    scale, -0 codes included): scale byte 0 and codes 0 for both, whatever the random
    bytes, and the rest of the tensor bit-exact."""
    B, R, Cc = 1, 64, 96
    rng = np.random.default_rng(23)
    codes4 = rng.integers(0, 16, size=(R, Cc), dtype=np.uint8)
    codes4[16:32, :] = rng.choice(np.array([0, 1, 8, 9], dtype=np.uint8), size=(16, Cc))
    codes4[16, :] = 1                                       # A = 2^-10 > 0 in every column
    codes4[48:64, :] = rng.choice(np.array([0, 8], dtype=np.uint8), size=(16, Cc))
    packed = (codes4[:, 0::2] | (codes4[:, 1::2] << 4)).astype(np.uint8).reshape(-1)
    scales = rng.integers(0x30, 0x50, size=(R, Cc // 16), dtype=np.uint8)
    scales[16:32, :] = 0x01                                 # 2^-9, the smallest E4M3 value
    c = torch.from_numpy(packed)
    s = torch.from_numpy(scales.reshape(-1).copy())
    ts = torch.ones(1, dtype=torch.float32)
    q = ops.NVFP4(c.to(DEV), s.to(DEV), ts.to(DEV), torch.zeros(B, device=DEV))
    for seed in range(3):
        t = ops.requant_transpose_sr(q, B, R, Cc, seed=seed)
        torch.cuda.synchronize()
        o = oracle.requant_transpose_sr(c, s, ts, B, R, Cc, seed)
        assert np.array_equal(npu8(t.codes), o["codes"]), f"seed {seed}"
        assert np.array_equal(npu8(t.scales), o["scales"]), f"seed {seed}"
        sc = npu8(t.scales).reshape(Cc, R // 16)
        cd = npu8(t.codes).reshape(Cc, R // 2)
        assert np.all(sc[:, 1] == 0) and np.all(sc[:, 3] == 0)
        assert np.all(cd[:, 8:16] == 0) and np.all(cd[:, 24:32] == 0)
        assert np.all(sc[:, 0] != 0)


def test_transpose_sr_64_seeds_unbiased():
    """All 64 seeds on a 1024x1024 tensor nearest-quantized from N(0,1): bit-exact
    against the oracle, and the mean over seeds of the requantized values tracks
    the exact transposed values up to the 8-bit resolution of the random bytes."""
    N = 1024
    x = inputs.transpose_source(N, N, device=DEV)
    q = ops.quantize(x)
    torch.cuda.synchronize()
    o = oracle.quantize(x.cpu(), 1, N, N)
    assert_q_equal(q, o, "1024^2")
    u = oracle.dequantize(o["codes"], o["scales"], np.ones(1, np.float32), 1, N, N).reshape(N, N).T
    acc = np.zeros((N, N))
    for seed in range(64):
        t = ops.requant_transpose_sr(q, 1, N, N, seed=seed)
        torch.cuda.synchronize()
        ot = oracle.requant_transpose_sr(o["codes"], o["scales"], o["tensor_scale"], 1, N, N, seed)
        assert np.array_equal(npu8(t.codes), ot["codes"]), f"seed {seed}"
        assert np.array_equal(npu8(t.scales), ot["scales"]), f"seed {seed}"
        acc += oracle.dequantize(ot["codes"], ot["scales"], np.ones(1, np.float32), 1, N,
                                 N).reshape(N, N)
    mean = acc / 64
    rel = (mean - u).sum() / np.abs(u).sum()
    assert abs(rel) < 2e-3, rel
    # Per-element expectation of the stochastic rounding in closed form: with
    # a = |y| between grid points G[lo] < a < G[lo+1] (spacing D), the step up is
    # taken for the ceil(256 p) bytes k < 256 p, p = (a - G[lo]) / D.  The signed,
    # standardised sum of (mean - expectation) over elements of each sign is a sum
    # of independent zero-mean terms, so a magnitude bias (for example truncation
    # toward zero, which cancels between the signs in the sum above) drives it far
    # from 0.
    G = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    dec = np.array([oracle.e4m3_value(b) for b in range(256)])[ot["scales"]].repeat(16)
    dec = dec.reshape(N, N)
    with np.errstate(divide="ignore"):
        rcp = np.where(dec > 0, (np.float32(1) / dec.astype(np.float32)), 0).astype(np.float32)
    y = (u.astype(np.float32) * rcp).astype(np.float32).astype(np.float64)
    a = np.abs(y)
    lo = np.clip(np.searchsorted(G, a, side="right") - 1, 0, 6)
    d = G[lo + 1] - G[lo]
    p = np.where(a >= 6, 0.0, (a - G[lo]) / d)
    pp = np.ceil(256 * p) / 256
    mag = np.where(a >= 6, 6.0, G[lo] + d * pp) * dec
    var = np.where(a >= 6, 0.0, (dec * d) ** 2 * pp * (1 - pp))
    sign = np.sign(y)
    expect = sign * mag
    assert np.all(mean[var == 0] == expect[var == 0]), "deterministic elements"
    for name, m in (("positive", sign > 0), ("negative", sign < 0), ("all", sign != 0)):
        z = (sign[m] * (mean[m] - expect[m])).sum() / np.sqrt(var[m].sum() / 64)
        assert abs(z) < 5, f"{name} elements: standardised magnitude deviation {z}"
    # below saturation the expectation exceeds |u| by less than one random-byte step,
    # D / 256 (up to the binary32 rounding of y = u * (1 / dec))
    ns = (a < 6) & (dec > 0)
    excess = (np.abs(expect) - np.abs(u))[ns]
    tol = 1e-6 * np.abs(u)[ns]
    assert np.all(excess >= -tol) and np.all(excess < (d * dec)[ns] / 256 + tol)


# ----------------------------------------------------------------------------------
# Grouped GEMM
# ----------------------------------------------------------------------------------

def _tile_rows(o, sample, seed):
    """Rows to check at full size: each group's first and last row, one random row of
    every 128-row block of every group (so every M-tile the kernel computes, including
    the interior tiles of the large groups, has a checked row; all N columns of a
    row are compared), and `sample` more random rows."""
    rng = np.random.default_rng(seed)
    M = int(o[-1])
    live = np.diff(o) > 0
    parts = [o[:-1][live], o[1:][live] - 1, rng.choice(M, sample, replace=False)]
    for g in range(len(o) - 1):
        for r0 in range(int(o[g]), int(o[g + 1]), 128):
            parts.append([rng.integers(r0, min(r0 + 128, int(o[g + 1])))])
    return np.unique(np.concatenate([np.asarray(p, np.int64) for p in parts]))


def _threaded_rows(fn, rows, threads=8):
    """fn(rows) -> (ref, asum) evaluated on row chunks in parallel host threads (the
    oracle's C routines release the GIL); results in row order."""
    from concurrent.futures import ThreadPoolExecutor
    chunks = [c for c in np.array_split(rows, threads) if c.size]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(fn, chunks))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def _gemm_check(counts, n, k, seed=5, sample=None, strict=True):
    """strict: |gpu - ref| <= 1e-3 * sum|a*w| (holds when |out| << sum|a*w|, as for the
    full-size random workloads).  Otherwise the bf16 rounding of the output is added:
    |bf16_rne(v) - v| <= 2^-8 |v|, so |gpu - ref| <= 1e-3 * sum|a*w| + 2^-8 (1 + 2^-7) |ref|
    (the fp32 accumulation error, below K * 2^-24 * sum|a*w|, fits in the first term)."""
    G = len(counts)
    M = int(sum(counts))
    a, w, off = inputs.grouped_gemm_inputs(groups=G, tokens=M, k=k, n=n, device="cpu", seed=seed,
                                           counts=counts)
    ow = oracle.quantize(w, G, n, k)
    wq = ops.NVFP4(torch.from_numpy(ow["codes"]).to(DEV), torch.from_numpy(ow["scales"]).to(DEV),
                   torch.from_numpy(ow["tensor_scale"]).to(DEV), torch.zeros(G, device=DEV))
    out = ops.grouped_gemm_nvfp4(a.to(DEV), off.to(DEV), wq, n, k)
    torch.cuda.synchronize()
    rows = np.arange(M) if sample is None else _tile_rows(off.numpy(), sample, seed)
    ref, asum = _threaded_rows(lambda r: oracle.grouped_gemm(
        a, off, n, k, ow["codes"], ow["scales"], ow["tensor_scale"], rows=r), rows)
    got = out.float().cpu().numpy()[rows].astype(np.float64)
    err = np.abs(got - ref)
    bound = 1e-3 * asum
    if not strict:
        bound = bound + 2.0 ** -8 * (1 + 2.0 ** -7) * np.abs(ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300))}"
    rb = torch.from_numpy(ref).to(torch.bfloat16).float().numpy()
    ulp = np.abs(got - rb) / np.maximum(np.spacing(np.abs(rb).astype(np.float32)) * 65536, 1e-300)
    return float(np.max(err / np.maximum(bound, 1e-300))), float(np.max(ulp))


def test_grouped_gemm_moe_full_size():
    """32 experts, Zipf(1.1) counts summing to 16384, K = 2048, N = 768."""
    counts = inputs.zipf_counts(32, 16384, 1.1)
    r, u = _gemm_check(counts, 768, 2048, sample=96)
    print(f"\ngrouped GEMM 32x[16384x2048x768]: max err/bound {r:.3e}, max bf16-ulp {u:.1f}")


def test_grouped_gemm_forward_shape():
    """64 experts, Zipf(1.1) counts summing to 16384, K = 768, N = 2048."""
    counts = inputs.zipf_counts(64, 16384, 1.1)
    r, u = _gemm_check(counts, 2048, 768, seed=6, sample=64)
    print(f"\ngrouped GEMM 64x[16384x768x2048]: max err/bound {r:.3e}, max bf16-ulp {u:.1f}")


GEMM_EDGES = [
    ([5, 0, 7, 1], 64, 64), ([1], 2, 16), ([130, 3], 66, 80), ([0, 0, 257], 200, 48),
    ([128, 128], 128, 128), ([64] * 5, 256, 2064), ([1, 2, 3, 4, 5, 6, 7], 130, 32),
    ([40, 300], 256, 1040), ([77], 128, 112),
    # more than 64 groups: the tile lookup walks the group offsets in chunks of 64
    ([(7 * g) % 23 if g % 5 else 0 for g in range(100)], 64, 96),
    ([(11 * g) % 37 for g in range(130)], 256, 64),
    # exactly 64 and 65 groups (one chunk, and one group into the second); n % 8 == 4
    ([3 + g % 4 for g in range(64)], 132, 48),
    ([g % 3 for g in range(65)], 40, 32),
]


@pytest.mark.parametrize("counts,n,k", GEMM_EDGES)
def test_grouped_gemm_edges(counts, n, k):
    _gemm_check(counts, n, k, strict=False)


# More shapes: one, two and three 64-wide K slices per tile, a single row, K far
# beyond the staged-scale limit (k = 12800, per-slice scale loads), ragged n, empty
# groups, one large group, and two mid-size problems with a ragged last column
# tile: [6000, 7000, 400, 3] x 520 (321 tiles, 8 columns in the last column tile)
# and [9000, 5000, 200] x 1032 (565 tiles, more than one round of the chip's 512
# workgroup slots).
GEMM_MORE = [
    ([8], 64, 64), ([5, 0, 7, 1], 64, 128), ([300, 1, 129], 136, 192), ([200], 256, 12800),
    ([0, 513, 0, 2], 520, 256), ([1000, 24, 3], 132, 640), ([4096], 768, 2048),
    ([6000, 7000, 400, 3], 520, 256), ([9000, 5000, 200], 1032, 192),
]


@pytest.mark.parametrize("counts,n,k", GEMM_MORE)
def test_grouped_gemm_more_shapes(counts, n, k):
    _gemm_check(counts, n, k, seed=9, sample=64 if sum(counts) > 2048 else None, strict=False)


def test_grouped_gemm_closed_form():
    """Small integers times W = 1 (code 2, scale 1.0, tensor scale 0.5): each output is
    half a row sum, exact in bf16."""
    G, n, k = 2, 64, 64
    counts = [3, 5]
    off = inputs.group_offsets(counts)
    A = (np.arange(8 * k).reshape(8, k) % 5 - 2).astype(np.float32)
    a = torch.from_numpy(A).to(torch.bfloat16)
    wq = ops.NVFP4(torch.full((G * n * k // 2,), 0x22, dtype=torch.uint8, device=DEV),
                   torch.full((G * n * k // 16,), 0x38, dtype=torch.uint8, device=DEV),
                   torch.tensor([0.5, 0.5], device=DEV), torch.zeros(G, device=DEV))
    out = ops.grouped_gemm_nvfp4(a.to(DEV), off.to(DEV), wq, n, k)
    torch.cuda.synchronize()
    want = 0.5 * A.sum(axis=1)[:, None] * np.ones((1, n))
    assert np.array_equal(out.float().cpu().numpy(), want)


# ----------------------------------------------------------------------------------
# Mismatch counting
# ----------------------------------------------------------------------------------

def _w4a4_check(counts, n, k, seed=7, sample=None, strict=True):
    """W4A4: the activations are nearest-quantized by the oracle (one tensor), the
    weights per expert; both NVFP4 operands go to the GPU and the result is checked
    against the oracle's float64 product of the decoded operands, to the bound of
    the bf16-activation GEMM."""
    G = len(counts)
    M = int(sum(counts))
    a, w, off = inputs.grouped_gemm_inputs(groups=G, tokens=M, k=k, n=n, device="cpu", seed=seed,
                                           counts=counts)
    oa = oracle.quantize(a, 1, M, k)
    ow = oracle.quantize(w, G, n, k)
    dev = lambda x: torch.from_numpy(x).to(DEV)
    aq = ops.NVFP4(dev(oa["codes"]), dev(oa["scales"]), dev(oa["tensor_scale"]),
                   torch.zeros(1, device=DEV))
    wq = ops.NVFP4(dev(ow["codes"]), dev(ow["scales"]), dev(ow["tensor_scale"]),
                   torch.zeros(G, device=DEV))
    out = ops.grouped_gemm_w4a4(aq, off.to(DEV), wq, n, k)
    torch.cuda.synchronize()
    rows = np.arange(M) if sample is None else _tile_rows(off.numpy(), sample, seed)
    ref, asum = _threaded_rows(lambda r: oracle.grouped_gemm_w4a4(
        oa["codes"], oa["scales"], oa["tensor_scale"], off, n, k, ow["codes"], ow["scales"],
        ow["tensor_scale"], rows=r), rows)
    got = out.float().cpu().numpy()[rows].astype(np.float64)
    err = np.abs(got - ref)
    bound = 1e-3 * asum
    if not strict:
        bound = bound + 2.0 ** -8 * (1 + 2.0 ** -7) * np.abs(ref)
    assert np.all(err <= bound), f"max err/bound {np.max(err / np.maximum(bound, 1e-300))}"


def test_w4a4_gemm_moe_full_size():
    _w4a4_check(inputs.zipf_counts(32, 16384, 1.1), 768, 2048, sample=256)


def test_w4a4_gemm_forward_shape():
    _w4a4_check(inputs.zipf_counts(64, 16384, 1.1), 2048, 768, sample=192)


@pytest.mark.parametrize("counts,n,k", GEMM_EDGES)
def test_w4a4_gemm_edges(counts, n, k):
    _w4a4_check(counts, n, k, strict=False)


@pytest.mark.parametrize("counts,n,k", GEMM_MORE[-2:])
def test_w4a4_gemm_mid_size(counts, n, k):
    """The two mid-size GEMM_MORE shapes for the W4A4 kernel."""
    _w4a4_check(counts, n, k, seed=11, sample=64, strict=False)


def test_grouped_gemms_repeatable():
    """Every output element of the full-size GEMMs, bit for bit, over repeated calls
    with the launches of other shapes in between.  The accumulation order is fixed
    by the kernel, so any difference between calls would come from a race on the
    activation tiles in LDS (written for a later slice while an earlier one is still
    read) or on the output staging."""
    shapes = [(inputs.zipf_counts(64, 16384, 1.1), 2048, 768),   # three LDS tiles
              (inputs.zipf_counts(32, 16384, 1.1), 768, 2048),   # three LDS tiles
              ([300, 1, 129, 700], 136, 784),                    # partial first slice
              ([64] * 5, 256, 2064)]                             # per-slice scale loads
    calls = []
    for i, (counts, n, k) in enumerate(shapes):
        G, M = len(counts), int(sum(counts))
        a, w, off = inputs.grouped_gemm_inputs(groups=G, tokens=M, k=k, n=n, device=DEV,
                                               seed=20 + i, counts=counts)
        wq = ops.quantize(w)  # [G, n, k]: one tensor scale per expert
        aq = ops.quantize(a)  # [M, k]: one tensor
        offd = off.to(DEV)
        calls.append((lambda a=a, offd=offd, wq=wq, n=n, k=k: ops.grouped_gemm_nvfp4(a, offd, wq, n, k),
                      f"bf16 {G}x[{M}x{k}x{n}]"))
        calls.append((lambda aq=aq, offd=offd, wq=wq, n=n, k=k: ops.grouped_gemm_w4a4(aq, offd, wq, n, k),
                      f"W4A4 {G}x[{M}x{k}x{n}]"))
    first = [f().view(torch.int16).clone() for f, _ in calls]
    torch.cuda.synchronize()
    for rep in range(6):
        for (f, name), ref in zip(calls if rep % 2 == 0 else calls[::-1],
                                  first if rep % 2 == 0 else first[::-1]):
            out = f()
            assert torch.equal(out.view(torch.int16), ref), f"{name}: call {rep + 2} differs"


@pytest.mark.parametrize("batch,per", [(3, 32 * (2 ** 20 + 7)), (64, 32 * 6149), (5, 32 * 9)])
def test_code_mismatch_ragged_and_capped(batch, per):
    """Mismatch counts over sizes that reach every path of the counting loop: pair
    counts (16 bytes of codes each) that leave a ragged last pass, whose extra loads
    are clamped to the last pair and not counted; a tensor of 2^20 + 7 pairs, more than
    its capped number of workgroups covers in one pass; several tensors per launch.
    Bit-exact against the oracle."""
    rng = np.random.default_rng(batch)
    a = rng.integers(0, 256, batch * per // 2, dtype=np.uint8)
    b = a.copy()
    flip = rng.random(b.size) < 0.01
    b[flip] ^= rng.integers(1, 256, int(flip.sum()), dtype=np.uint8)
    # the last pair of every tensor differs, so that a clamped load counted twice would show
    last = np.arange(1, batch + 1) * (per // 2) - 1
    b[last] = a[last] ^ 0x11
    got = ops.code_mismatch(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV), batch, per)
    torch.cuda.synchronize()
    want = oracle.code_mismatch(a, b, batch, per)
    assert np.array_equal(got.cpu().numpy().astype(np.uint64), want)
    assert (want[:, 0] > 0).all()


def test_code_mismatch_random():
    rng = np.random.default_rng(3)
    B, per = 5, 4096
    a = rng.integers(0, 256, B * per // 2, dtype=np.uint8)
    b = a.copy()
    flip = rng.random(b.size) < 0.05
    b[flip] = rng.integers(0, 256, flip.sum(), dtype=np.uint8)
    got = ops.code_mismatch(torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV), B, per)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().astype(np.uint64), oracle.code_mismatch(a, b, B, per))

"""Benchmark of the block-scaled FP4 hot path on one MI355X.

One step = the whole path over the MoE expert-weights workload: 48 layers x 64
experts x [2048 x 768] bf16 weights, a rollout copy X_r and a training copy
X_t, both resident in HBM.  The step runs in phases, each one kernel over all
48 layers:

  1. tensor amax of X_r (per expert)
  2. rollout nearest quantize of X_r; for the latter half of the layers the
     packed 1-bit hint is emitted in the same pass
  3. tensor amax of X_t, trainer nearest quantize of X_t (unguided baseline)
  4. trainer guided quantize of X_t with the hints (latter half of the layers)
  5. code-mismatch counts rollout vs trainer (before / after guidance)
  6. dequantize -> transpose -> stochastic-rounding requantize of the trainer's
     weights (the backward copy), Philox seed = layer
  7. grouped GEMM: 16384 bf16 token rows, Zipf(1.1) over the 64 experts, times
     the trainer's NVFP4 weights (K = 768, N = 2048), bf16 out

`value` is the step's algorithmic bytes (every input read once, every output
written once) over the measured step time, in GB/s.  Per-kernel durations
come from HIP events recorded on the launch stream around each phase of the
timed steps (phase time / launches).  The CPU oracle is timed on a bounded
sample of the same work.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2]
"""
from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0

LAYERS, EXPERTS, ROWS, COLS = 48, 64, 2048, 768
TOKENS = 16384


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the rows measured outside the step (W4A4 GEMM, FP4 KV cache)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path has no "
                                   "multi-GPU leg (--gpus must be 1)"}))
        sys.exit(2)

    import numpy as np
    import torch

    from fp4_quantization_precision_amd import _lib, inputs, ops
    from fp4_quantization_precision_amd._lib import TQ_AMAX_GIVEN, TQ_BF16

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = _lib.lib()
    stream = torch.cuda.current_stream()
    sp = C.c_void_p(stream.cuda_stream)
    P = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None

    nl = args.layers
    first_hint = ops.hint_first_layer(LAYERS)
    per = ROWS * COLS
    n_layer = EXPERTS * per

    # ---------------- inputs resident in HBM ----------------
    t_gen = time.perf_counter()
    XR = torch.empty((nl, EXPERTS, ROWS, COLS), dtype=torch.bfloat16, device=dev)
    XT = torch.empty_like(XR)
    for l in range(nl):
        xr, xt = inputs.moe_expert_weights_layer(l, EXPERTS, ROWS, COLS, device=dev)
        XR[l].copy_(xr)
        XT[l].copy_(xt)
        del xr, xt
    counts = inputs.zipf_counts(EXPERTS, TOKENS, 1.1)
    OFF = inputs.group_offsets(counts).to(dev)
    gA = torch.Generator(device=dev)
    gA.manual_seed(5)
    A = torch.randn((nl, TOKENS, COLS), generator=gA, device=dev).to(torch.bfloat16)
    torch.cuda.synchronize()
    t_gen = time.perf_counter() - t_gen

    # ---------------- outputs ----------------
    def q_bufs():
        return ops.NVFP4(torch.empty((nl, EXPERTS, ROWS, COLS // 2), dtype=torch.uint8, device=dev),
                         torch.empty((nl, EXPERTS, ROWS, COLS // 16), dtype=torch.uint8, device=dev),
                         torch.empty((nl, EXPERTS), dtype=torch.float32, device=dev),
                         torch.empty((nl, EXPERTS), dtype=torch.float32, device=dev))
    QR, QN, QG = q_bufs(), q_bufs(), q_bufs()
    nh = max(nl - first_hint, 0)
    H = torch.empty((max(nh, 1), ops.hint_words(n_layer)), dtype=torch.int32, device=dev)
    CNT = torch.empty((2, nl, EXPERTS, 2), dtype=torch.int64, device=dev)  # [nearest|guided]
    QT = ops.NVFP4(torch.empty((nl, EXPERTS, COLS, ROWS // 2), dtype=torch.uint8, device=dev),
                   torch.empty((nl, EXPERTS, COLS, ROWS // 16), dtype=torch.uint8, device=dev),
                   torch.empty((nl, EXPERTS), dtype=torch.float32, device=dev), None)
    OUT = torch.empty((nl, TOKENS, ROWS), dtype=torch.bfloat16, device=dev)

    # ---------------- pre-bound calls (validated once by the library) ----------------
    # The step runs as phases, each one kind of kernel: the rollout's amax and
    # quantize (with hints for the latter half), the trainer's amax, nearest and
    # guided quantize, the mismatch counts, the SR transpose and the grouped GEMM.
    # The layers' tensors are contiguous, so the streaming phases cover all the
    # layers they apply to in one call (a batch of layers x experts tensors);
    # the grouped GEMM runs once per layer.  Events bracket each phase, so the
    # per-kernel averages carry no per-call event overhead.
    phases = {}  # phase name -> list of (category, fn, args, layers covered)

    def add(phase, cat, fn, a, layers):
        phases.setdefault(phase, []).append((cat, fn, a, layers))

    fh, E = first_hint, EXPERTS
    add("amax_rollout", "amax", L.tq_tensor_amax,
        (P(XR), TQ_BF16, nl * E, per, P(QR.tensor_amax), sp), nl)
    if fh > 0:
        add("quantize_rollout", "quantize", L.tq_quantize,
            (P(XR[0]), TQ_BF16, fh * E, ROWS, COLS, P(QR.tensor_amax[0]), P(QR.codes[0]),
             P(QR.scales[0]), P(QR.tensor_scale[0]), None, TQ_AMAX_GIVEN, sp), fh)
    if nh > 0:
        add("quantize_hint_rollout", "quantize_hint", L.tq_quantize,
            (P(XR[fh]), TQ_BF16, nh * E, ROWS, COLS, P(QR.tensor_amax[fh]), P(QR.codes[fh]),
             P(QR.scales[fh]), P(QR.tensor_scale[fh]), P(H), TQ_AMAX_GIVEN, sp), nh)
    add("amax_trainer", "amax", L.tq_tensor_amax,
        (P(XT), TQ_BF16, nl * E, per, P(QN.tensor_amax), sp), nl)
    add("quantize_trainer", "quantize", L.tq_quantize,
        (P(XT), TQ_BF16, nl * E, ROWS, COLS, P(QN.tensor_amax), P(QN.codes), P(QN.scales),
         P(QN.tensor_scale), None, TQ_AMAX_GIVEN, sp), nl)
    if nh > 0:
        add("guided_trainer", "guided", L.tq_quantize_guided,
            (P(XT[fh]), TQ_BF16, nh * E, ROWS, COLS, P(QN.tensor_amax[fh]), P(H),
             P(QG.codes[fh]), P(QG.scales[fh]), P(QG.tensor_scale[fh]), TQ_AMAX_GIVEN, sp), nh)
    add("mismatch", "mismatch", L.tq_code_mismatch,
        (P(QR.codes), P(QN.codes), nl * E, per, P(CNT[0]), sp), nl)
    if nh > 0:
        add("mismatch", "mismatch", L.tq_code_mismatch,
            (P(QR.codes[fh]), P(QG.codes[fh]), nh * E, per, P(CNT[1, fh]), sp), nh)
    # the backward copy of the trainer's weights: unguided layers from QN, hinted
    # ones from QG (Philox seed 0 and 1; the counter runs over each call's elements)
    if fh > 0:
        add("sr_transpose", "sr_transpose", L.tq_requant_transpose_sr,
            (P(QN.codes[0]), P(QN.scales[0]), P(QN.tensor_scale[0]), fh * E, ROWS, COLS,
             C.c_uint64(0), P(QT.codes[0]), P(QT.scales[0]), P(QT.tensor_scale[0]), sp), fh)
    if nh > 0:
        add("sr_transpose", "sr_transpose", L.tq_requant_transpose_sr,
            (P(QG.codes[fh]), P(QG.scales[fh]), P(QG.tensor_scale[fh]), nh * E, ROWS, COLS,
             C.c_uint64(1), P(QT.codes[fh]), P(QT.scales[fh]), P(QT.tensor_scale[fh]), sp), nh)
    for l in range(nl):
        trainer = QG if l >= fh else QN
        add("gemm", "gemm", L.tq_grouped_gemm_nvfp4,
            (P(A[l]), P(OFF), EXPERTS, TOKENS, ROWS, COLS, P(trainer.codes[l]),
             P(trainer.scales[l]), P(trainer.tensor_scale[l]), P(OUT[l]), sp), 1)
    calls = [c for ph in phases.values() for c in ph]

    # algorithmic bytes per layer covered (inputs read once + outputs written once)
    def layer_bytes(cat):
        n = n_layer
        return {
            "amax": 2.0 * n,
            "quantize": n * (2 + 0.5 + 1 / 16),
            "quantize_hint": n * (2 + 0.5 + 1 / 16 + 1 / 8),
            "guided": n * (2 + 1 / 8 + 0.5 + 1 / 16),
            "mismatch": n * (0.5 + 0.5),
            "sr_transpose": n * 2 * (0.5 + 1 / 16),
            "gemm": TOKENS * COLS * 2 + n * (0.5 + 1 / 16) + TOKENS * ROWS * 2,
        }[cat]
    gemm_flops = 2.0 * TOKENS * COLS * ROWS
    step_bytes = sum(layer_bytes(c) * nlay for c, _, _, nlay in calls)
    step_flops = gemm_flops * nl

    def run_step(events=None):
        for name, ph in phases.items():
            if events is not None:
                events[name][0].record(stream)
            for cat, fn, a, _ in ph:
                st = fn(*a)
                if st != 0:
                    raise RuntimeError(f"{cat}: {L.tq_status_string(st).decode()}")
            if events is not None:
                events[name][1].record(stream)

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()

    # ---------------- timed steps ----------------
    new_ev = lambda: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev = [{name: new_ev() for name in phases} for _ in range(args.steps)]
    step_ev = [new_ev() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step_ev[s][0].record(stream)
        run_step(ev[s])
        step_ev[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps
    ev_step_ms = float(np.mean([a.elapsed_time(b) for a, b in step_ev]))

    # per category: phase time summed over the timed steps / launches; bytes per
    # launch = the category's algorithmic bytes per step / its launches per step
    cat_ms, cat_n, cat_layers = {}, {}, {}
    for name, ph in phases.items():
        cat = ph[0][0]
        cat_n[cat] = cat_n.get(cat, 0) + len(ph)
        cat_layers[cat] = cat_layers.get(cat, 0) + sum(c[3] for c in ph)
        for s in range(args.steps):
            cat_ms[cat] = cat_ms.get(cat, 0.0) + ev[s][name][0].elapsed_time(ev[s][name][1])

    def call_bytes(cat):  # average algorithmic bytes per launch of a category
        return layer_bytes(cat) * cat_layers[cat] / cat_n[cat]
    kernels = {}
    for cat in cat_ms:
        us = 1e3 * cat_ms[cat] / (cat_n[cat] * args.steps)
        ent = {"launches_per_step": cat_n[cat], "layers_per_launch": cat_layers[cat] / cat_n[cat],
               "avg_us": round(us, 2)}
        if cat == "gemm":
            ent["TFLOP/s"] = round(gemm_flops / (us * 1e-6) / 1e12, 1)
            ent["frac_bf16_mfma_peak"] = round(ent["TFLOP/s"] / BF16_MFMA_PEAK_TFLOPS, 4)
        ent["GB/s"] = round(call_bytes(cat) / (us * 1e-6) / 1e9, 1)
        ent["frac_hbm_peak"] = round(ent["GB/s"] / HBM_PEAK_GBS, 4)
        ent["share_of_step"] = round(cat_ms[cat] / args.steps / ev_step_ms, 4)
        kernels[cat] = ent

    # mismatch statistics of the last step
    cnt = CNT.sum(dim=2).cpu().numpy()  # [nearest|guided, layer, (mismatches, adjacent)]
    mism = {"nearest_rate": float(cnt[0, :, 0].sum() / (nl * n_layer)),
            "nearest_adjacent_frac": float(cnt[0, :, 1].sum() / max(cnt[0, :, 0].sum(), 1))}
    if nh:
        mism["hinted_layers_nearest_rate"] = float(cnt[0, first_hint:, 0].sum() / (nh * n_layer))
        mism["hinted_layers_guided_rate"] = float(cnt[1, first_hint:, 0].sum() / (nh * n_layer))

    if args.copy_calibration:
        # one plain device copy of 1 GiB (read 1 GiB, write 1 GiB): the yardstick
        # for the HBM byte counters (FETCH_SIZE / WRITE_SIZE) of the kernels above
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # the roofline is reported for the kernel with the largest share of the step
    dom_cat = max(kernels, key=lambda c: kernels[c]["share_of_step"])
    dom = kernels[dom_cat]
    kname = KERNEL_OF[dom_cat][0]
    if dom_cat == "gemm":
        roofline = {"bound": "mfma", "achieved": dom["TFLOP/s"], "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": dom["frac_bf16_mfma_peak"]}
    else:
        roofline = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dom["frac_hbm_peak"]}
    roofline.update({"traffic": measured_traffic(dom_cat, dom["layers_per_launch"]),
                     "kernel": kname, "category": dom_cat,
                     "algorithmic_bytes_per_launch": call_bytes(dom_cat),
                     "avg_launch_us": dom["avg_us"], "share_of_step": dom["share_of_step"]})
    if dom_cat == "gemm":
        roofline["algorithmic_flops_per_launch"] = gemm_flops

    extras = None if args.no_extras else measure_extras(L, dev, stream, A, OFF, QG, QN, nl, first_hint)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(XR, XT, A, counts, first_hint)

    line = {
        "metric": "quantize/guided-quantize GB/s and % of HBM peak; grouped-GEMM TFLOP/s",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"moe-expert-weights {nl}x{EXPERTS}x[{ROWS}x{COLS}] bf16 "
                               f"(rollout+trainer copies; hints for layers >= {first_hint}; "
                               f"SR transpose; grouped GEMM {TOKENS} tokens/layer)",
                   "layers": nl, "experts": EXPERTS, "rows": ROWS, "cols": COLS,
                   "gemm_tokens_per_layer": TOKENS, "gemm_k": COLS, "gemm_n": ROWS,
                   "parallelism": "single GPU"},
        "step_bytes": step_bytes,
        "step_gemm_tflops": round(step_flops / (ms_per_step * 1e-3) / 1e12, 1),
        "event_ms_per_step": round(ev_step_ms, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "extras": extras,
        "mismatch": mism,
        "input_generation_s": round(t_gen, 1),
    }
    print(json.dumps(line), flush=True)


def _time_phase(stream, fn, reps):
    """Average event time (us) of `reps` back-to-back calls of fn on `stream`."""
    import torch
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def measure_extras(L, dev, stream, A, OFF, QG, QN, nl, first_hint):
    """Rows measured outside the step, on the same device buffers:
    * W4A4 grouped GEMM: each layer's activations quantized to NVFP4 (one tensor),
      then the GEMM with the trainer's NVFP4 weights;
    * FP4 KV cache with hints: one layer's K and V cache [32768 x 8 x 128] bf16,
      rollout nearest + hints and trainer guided, per token-head blocks of 16;
    * 16x16-tile scaling: quantize and exact transpose of the activations
      workload [32768 x 4096] bf16, and the share of zero codes against block-16;
    * MXFP8 for the backward: nearest quantize of the activations workload and the
      NVFP4 -> MXFP8 stochastic-rounding transpose of each layer's trainer weights;
    * the grouped GEMM at 32 experts, 16384 tokens, K = 2048, N = 768."""
    import ctypes as C

    import torch

    from fp4_quantization_precision_amd import inputs, ops
    from fp4_quantization_precision_amd._lib import TQ_BF16

    sp = C.c_void_p(stream.cuda_stream)
    P = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
    out = {}

    # ---- W4A4 grouped GEMM ----
    AQ = [ops.new_nvfp4((1,), TOKENS, COLS, dev) for _ in range(nl)]
    OUT = torch.empty((TOKENS, ROWS), dtype=torch.bfloat16, device=dev)

    def quant_a():
        for l in range(nl):
            st = L.tq_quantize(P(A[l]), TQ_BF16, 1, TOKENS, COLS, P(AQ[l].tensor_amax), P(AQ[l].codes),
                               P(AQ[l].scales), P(AQ[l].tensor_scale), None, 0, sp)
            assert st == 0

    def w4a4():
        for l in range(nl):
            w = QG if l >= first_hint else QN
            st = L.tq_grouped_gemm_w4a4(P(AQ[l].codes), P(AQ[l].scales), P(AQ[l].tensor_scale),
                                        P(OFF), EXPERTS, TOKENS, ROWS, COLS, P(w.codes[l]),
                                        P(w.scales[l]), P(w.tensor_scale[l]), P(OUT), sp)
            assert st == 0

    us_q = _time_phase(stream, quant_a, 3) / nl
    us_g = _time_phase(stream, w4a4, 3) / nl
    flops = 2.0 * TOKENS * COLS * ROWS
    n_a = TOKENS * COLS
    out["w4a4_quantize_activations"] = {
        "kernel": "tq::amax_kernel + tq::quantize_kernel (tq_quantize, batch 1)",
        "avg_us": round(us_q, 2), "GB/s": round(n_a * (2 + 2 + 0.5625) / us_q / 1e3, 1),
        "note": "amax pass + quantize pass over [16384 x 768] bf16 per layer"}
    out["w4a4_gemm"] = {
        "kernel": "tq::grouped_gemm_nvfp4_kernel<true>", "avg_us": round(us_g, 2),
        "TFLOP/s": round(flops / us_g / 1e6, 1),
        "frac_bf16_mfma_peak": round(flops / us_g / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4),
        "shape": f"{EXPERTS} experts, {TOKENS} tokens, K {COLS}, N {ROWS}"}
    del AQ, OUT

    # ---- grouped GEMM at its own configuration: 32 experts, Zipf(1.1) token
    # counts summing to 16384, K = 2048, N = 768; four input sets rotate so that
    # the timed calls do not run from the 256 MB Infinity Cache ----
    G5, T5, K5, N5 = 32, 16384, 2048, 768
    sets5 = []
    for i in range(4):
        a5, w5, off5 = inputs.grouped_gemm_inputs(G5, T5, K5, N5, device=dev, seed=5 + i)
        sets5.append((a5, ops.quantize(w5), off5.to(dev)))
        del w5
    out5 = torch.empty((T5, N5), dtype=torch.bfloat16, device=dev)

    def gemm_c5():
        for a5, q5, off5 in sets5:
            st = L.tq_grouped_gemm_nvfp4(P(a5), P(off5), G5, T5, N5, K5, P(q5.codes), P(q5.scales),
                                         P(q5.tensor_scale), P(out5), sp)
            assert st == 0

    us5 = _time_phase(stream, gemm_c5, 5) / len(sets5)
    flops5 = 2.0 * T5 * K5 * N5
    out["gemm_32_experts"] = {
        "kernel": "tq::grouped_gemm_nvfp4_kernel", "avg_us": round(us5, 2),
        "TFLOP/s": round(flops5 / us5 / 1e6, 1),
        "frac_bf16_mfma_peak": round(flops5 / us5 / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4),
        "shape": f"{G5} experts, {T5} tokens, K {K5}, N {N5}, Zipf(1.1) counts"}
    del sets5, out5

    # ---- FP4 KV cache with hints ----
    T, Hh, D = 32768, 8, 128
    kr, kt, vr, vt, _ = inputs.kv_cache(T, Hh, D, device=dev)
    R, n = T * Hh, T * Hh * D
    H = torch.empty(2, ops.hint_words(n), dtype=torch.int32, device=dev)
    QR = [ops.new_nvfp4((1,), R, D, dev) for _ in range(2)]
    QT = [ops.new_nvfp4((1,), R, D, dev) for _ in range(2)]
    xs_r, xs_t = (kr, vr), (kt, vt)
    for i in range(2):  # trainer amax (given to the guided quantizer, as in the step)
        assert L.tq_tensor_amax(P(xs_t[i]), TQ_BF16, 1, n, P(QT[i].tensor_amax), sp) == 0

    def kv_hint():
        for i in range(2):
            st = L.tq_quantize(P(xs_r[i]), TQ_BF16, 1, R, D, P(QR[i].tensor_amax), P(QR[i].codes),
                               P(QR[i].scales), P(QR[i].tensor_scale), P(H[i]), 0, sp)
            assert st == 0

    def kv_guided():
        for i in range(2):
            st = L.tq_quantize_guided(P(xs_t[i]), TQ_BF16, 1, R, D, P(QT[i].tensor_amax), P(H[i]),
                                      P(QT[i].codes), P(QT[i].scales), P(QT[i].tensor_scale), 1, sp)
            assert st == 0

    us_h = _time_phase(stream, kv_hint, 5) / 2
    us_gd = _time_phase(stream, kv_guided, 5) / 2
    out["kv_quantize_hint"] = {
        "kernel": "tq::amax_kernel + tq::quantize_kernel<true, 1>", "avg_us": round(us_h, 2),
        "GB/s": round(n * (2 + 2 + 0.6875) / us_h / 1e3, 1),
        "note": "per K or V tensor [32768 x 8 x 128]: amax pass + quantize with hints"}
    out["kv_guided"] = {
        "kernel": "tq::quantize_kernel<true, 2>", "avg_us": round(us_gd, 2),
        "GB/s": round(n * 2.6875 / us_gd / 1e3, 1),
        "frac_hbm_peak": round(n * 2.6875 / us_gd / 1e3 / HBM_PEAK_GBS, 4)}
    # ---- MXFP8 backward: nearest quantize of activations, NVFP4 -> MXFP8 SR transpose ----
    T3, H3 = 32768, 4096
    xm, _, _ = inputs.activations(T3, H3, device=dev)
    n3 = T3 * H3
    mxc = torch.empty((T3, H3), dtype=torch.uint8, device=dev)
    mxs = torch.empty((T3, H3 // 32), dtype=torch.uint8, device=dev)

    def mx_quant():
        assert L.tq_quantize_mxfp8(P(xm), TQ_BF16, 1, T3, H3, P(mxc), P(mxs), sp) == 0

    per = ROWS * COLS
    mct = torch.empty((EXPERTS, COLS, ROWS), dtype=torch.uint8, device=dev)
    mst = torch.empty((EXPERTS, COLS, ROWS // 32), dtype=torch.uint8, device=dev)
    mts = torch.empty(EXPERTS, dtype=torch.float32, device=dev)

    def mx_transpose():
        for l in range(nl):
            w = QG if l >= first_hint else QN
            assert L.tq_requant_transpose_mxfp8_sr(P(w.codes[l]), P(w.scales[l]), P(w.tensor_scale[l]),
                                                   EXPERTS, ROWS, COLS, C.c_uint64(l), P(mct), P(mst),
                                                   P(mts), sp) == 0

    us_mq = _time_phase(stream, mx_quant, 5)
    us_mt = _time_phase(stream, mx_transpose, 2) / nl
    b_mq = n3 * (2 + 1 + 1 / 32)
    b_mt = EXPERTS * per * (0.5625 + 1 + 1 / 32)
    out["mxfp8_quantize"] = {
        "kernel": "tq::quantize_mxfp8_kernel<true>", "avg_us": round(us_mq, 2),
        "GB/s": round(b_mq / us_mq / 1e3, 1), "frac_hbm_peak": round(b_mq / us_mq / 1e3 / HBM_PEAK_GBS, 4),
        "workload": f"activations [{T3} x {H3}] bf16"}
    out["mxfp8_sr_transpose"] = {
        "kernel": "tq::requant_transpose_mxfp8_sr_kernel", "avg_us": round(us_mt, 2),
        "GB/s": round(b_mt / us_mt / 1e3, 1), "frac_hbm_peak": round(b_mt / us_mt / 1e3 / HBM_PEAK_GBS, 4),
        "workload": f"one MoE layer of trainer NVFP4 weights {EXPERTS} x [{ROWS} x {COLS}] -> MXFP8 [{COLS} x {ROWS}]"}
    del xm, mxc, mxs, mct, mst, mts

    # ---- 16x16-tile scaling on the activations workload ----
    T2, Hd = 32768, 4096
    xa, _, _ = inputs.activations(T2, Hd, device=dev)
    n2 = T2 * Hd
    q16 = ops.quantize_tile16(xa)
    qt16 = ops.transpose_tile16(q16, 1, T2, Hd)

    def tile_quant():
        assert L.tq_quantize_tile16(P(xa), TQ_BF16, 1, T2, Hd, P(q16.tensor_amax), P(q16.codes),
                                    P(q16.scales), P(q16.tensor_scale), 1, sp) == 0

    def tile_transpose():
        assert L.tq_transpose_tile16(P(q16.codes), P(q16.scales), P(q16.tensor_scale), 1, T2, Hd,
                                     P(qt16.codes), P(qt16.scales), P(qt16.tensor_scale), sp) == 0

    us_tq = _time_phase(stream, tile_quant, 5)
    us_tt = _time_phase(stream, tile_transpose, 5)
    b_tq = n2 * (2 + 0.5 + 1 / 256)
    b_tt = n2 * 2 * (0.5 + 1 / 256)
    qb = ops.quantize(xa)
    zero16 = ((q16.codes & 0x07) == 0).sum() + ((q16.codes & 0x70) == 0).sum()
    zerob = ((qb.codes & 0x07) == 0).sum() + ((qb.codes & 0x70) == 0).sum()
    nz = (xa != 0).sum()
    out["tile16_quantize"] = {
        "kernel": "tq::quantize_tile16_kernel<true>", "avg_us": round(us_tq, 2),
        "GB/s": round(b_tq / us_tq / 1e3, 1), "frac_hbm_peak": round(b_tq / us_tq / 1e3 / HBM_PEAK_GBS, 4),
        "workload": f"activations [{T2} x {Hd}] bf16, amax given"}
    out["tile16_transpose"] = {
        "kernel": "tq::transpose_tile16_kernel", "avg_us": round(us_tt, 2),
        "GB/s": round(b_tt / us_tt / 1e3, 1), "frac_hbm_peak": round(b_tt / us_tt / 1e3 / HBM_PEAK_GBS, 4)}
    out["tile16_vs_block16_zeroed"] = {
        "tile16_zero_codes_frac": float(zero16) / n2, "block16_zero_codes_frac": float(zerob) / n2,
        "nonzero_inputs_frac": float(nz) / n2}
    del xa, q16, qt16, qb

    cnt = torch.empty(2, 2, dtype=torch.int64, device=dev)
    qn = ops.quantize(kt.view(1, R, D))
    ops.code_mismatch(torch.cat([QR[0].codes.reshape(-1)] * 2),
                      torch.cat([qn.codes.reshape(-1), QT[0].codes.reshape(-1)]), 2, n, counts=cnt)
    c = cnt.cpu().numpy()
    out["kv_mismatch_K"] = {"nearest_rate": float(c[0, 0] / n), "guided_rate": float(c[1, 0] / n),
                            "nearest_adjacent_frac": float(c[0, 1] / max(c[0, 0], 1))}
    return out


# kernel name and source file of each timed category
KERNEL_OF = {
    "amax": ("tq::amax_kernel<true>", "tq_quantize.hip"),
    "quantize": ("tq::quantize_kernel<true, 0>", "tq_quantize.hip"),
    "quantize_hint": ("tq::quantize_kernel<true, 1>", "tq_quantize.hip"),
    "guided": ("tq::quantize_kernel<true, 2>", "tq_quantize.hip"),
    "mismatch": ("tq::mismatch_kernel", "tq_quantize.hip"),
    "sr_transpose": ("tq::requant_transpose_sr_kernel", "tq_sr.hip"),
    "gemm": ("tq::grouped_gemm_nvfp4_kernel", "tq_gemm.hip"),
}

# HBM bytes per layer covered, from rocprofv3 FETCH_SIZE and WRITE_SIZE passes
# over this benchmark (KiB per dispatch scaled by what the same counters read for
# the 1 GiB device copy of --copy-calibration, divided by the layers the
# dispatch covers), keyed by the SHA-256 of the kernel's source and the shared
# device header: a figure is reported only for the code it was measured on.
TRAFFIC = {
    # FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0: the 1 GiB copy read 524314 KiB fetched and
    # 1048576 KiB written.  Ratio to the algorithmic bytes in the comments.
    "amax": {"bytes_per_layer": 201325797, "fetch_kib": 4718757.1, "write_kib": 96.0, "layers": 48, "sources_sha256": "219cc3dce9ba5a108375d338a1ab9131292a3111e54af0e89ed55b8b9ad46fdd"},  # 1.000
    "quantize": {"bytes_per_layer": 257944055, "fetch_kib": 3538979.9, "write_kib": 1990733.5, "layers": 36, "sources_sha256": "219cc3dce9ba5a108375d338a1ab9131292a3111e54af0e89ed55b8b9ad46fdd"},  # 1.000
    "quantize_hint": {"bytes_per_layer": 270528010, "fetch_kib": 2359332.4, "write_kib": 1622067.1, "layers": 24, "sources_sha256": "219cc3dce9ba5a108375d338a1ab9131292a3111e54af0e89ed55b8b9ad46fdd"},  # 1.000
    "guided": {"bytes_per_layer": 270530639, "fetch_kib": 2506847.8, "write_kib": 1327112.6, "layers": 24, "sources_sha256": "219cc3dce9ba5a108375d338a1ab9131292a3111e54af0e89ed55b8b9ad46fdd"},  # 1.000
    "mismatch": {"bytes_per_layer": 101033841, "fetch_kib": 1769513.6, "write_kib": 13117.7, "layers": 36, "sources_sha256": "219cc3dce9ba5a108375d338a1ab9131292a3111e54af0e89ed55b8b9ad46fdd"},  # 1.004
    "sr_transpose": {"bytes_per_layer": 135414149, "fetch_kib": 674280.6, "write_kib": 1825274.2, "layers": 24, "sources_sha256": "eac8271f5410576433458a8d725da328e8b742bdd99a233b77055ff5c6fc8f42"},  # 1.196
    "gemm": {"bytes_per_layer": 159250907, "fetch_kib": 44993.4, "write_kib": 65536.0, "layers": 1, "sources_sha256": "234bcd5a07abdf64d459419c0990277f1f94565dcccbe9d323ff0f877f428939"},  # 1.070
}


def _sources_digest(src):
    import hashlib
    h = hashlib.sha256()
    for f in (src, "tq_device.hpp"):
        with open(os.path.join(ROOT, "fp4_quantization_precision_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(cat, layers_per_launch):
    """Counter-measured HBM bytes per launch of `cat`, or None if not measured on
    the current sources."""
    ent = TRAFFIC.get(cat)
    if ent is None or _sources_digest(KERNEL_OF[cat][1]) != ent["sources_sha256"]:
        return None
    return round(ent["bytes_per_layer"] * layers_per_launch)


def cpu_baseline(XR, XT, A, counts, first_hint):
    """The CPU oracle on a bounded sample of one step: experts 0 and 1 of layer
    `first_hint` (a hinted layer) through amax, nearest (rollout + trainer),
    hints, guided, mismatch counts and the SR transpose, plus the grouped-GEMM
    rows of the same share of the layer's tokens (2/64 of 16384 rows), scaled to
    GB/s with the same algorithmic bytes as the GPU step."""
    import numpy as np

    import oracle
    l, ne = first_hint, 2
    per = ROWS * COLS
    xr = XR[l, :ne].cpu()
    xt = XT[l, :ne].cpu()
    a = A[l].cpu()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    rows = np.arange(0, TOKENS, 16)[: 2 * TOKENS * ne // EXPERTS]  # 1024 token rows spread over the layer
    t0 = time.perf_counter()
    qr = oracle.quantize(xr, ne, ROWS, COLS)
    h = oracle.extract_hint(qr["codes"], ne * per)
    qn = oracle.quantize(xt, ne, ROWS, COLS)
    qg = oracle.quantize_guided(xt, ne, ROWS, COLS, h, amax=qn["tensor_amax"])
    oracle.code_mismatch(qr["codes"], qn["codes"], ne, per)
    oracle.code_mismatch(qr["codes"], qg["codes"], ne, per)
    oracle.requant_transpose_sr(qg["codes"], qg["scales"], qg["tensor_scale"], ne, ROWS, COLS, l)
    t_q = time.perf_counter() - t0
    # GEMM rows need every expert's weights: quantize the trainer weights of all
    # experts with the GPU-independent oracle first (not timed: it is the
    # quantize step, already sampled above), then time the rows.
    wq = oracle.quantize(XT[l].cpu(), EXPERTS, ROWS, COLS)
    t1 = time.perf_counter()
    oracle.grouped_gemm(a, off, ROWS, COLS, wq["codes"], wq["scales"], wq["tensor_scale"], rows=rows)
    t_g = time.perf_counter() - t1
    n = ne * per
    q_bytes = n * (2.0 * 2 + (2 + 0.5 + 1 / 16 + 1 / 8) + (2 + 0.5 + 1 / 16) + (2 + 1 / 8 + 0.5 + 1 / 16)
                   + 2 * 1.0 + 2 * (0.5 + 1 / 16))
    g_bytes = (TOKENS * COLS * 2 + EXPERTS * per * (0.5 + 1 / 16) + TOKENS * ROWS * 2) * rows.size / TOKENS
    secs = t_q + t_g
    return {"value": round((q_bytes + g_bytes) / secs / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"layer {l}, experts 0-1 ({n} weights): amax, nearest x2, hints, guided, "
                      f"mismatch x2, SR transpose ({t_q:.1f} s); grouped-GEMM fp64 rows "
                      f"{rows.size}/{TOKENS} of the layer ({t_g:.1f} s)",
            "seconds": round(secs, 2)}


if __name__ == "__main__":
    main()

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
     weights (the backward copy), Philox seed 0 for the unguided layers and 1
     for the hinted ones
  7. grouped GEMM: 16384 bf16 token rows, Zipf(1.1) over the 64 experts, times
     the trainer's NVFP4 weights (K = 768, N = 2048), bf16 out

`value` is the step's algorithmic bytes (every input read once, every output
written once) over the measured step time, in GB/s.  Per-kernel durations
come from HIP events recorded on the launch stream around each phase of the
timed steps (phase time / launches).

`configs` holds one row per workload configuration (tiny round trip,
activations 32768 x 4096, transpose-requantize 8192^2 per seed, grouped GEMM
32 experts x K 2048 x N 768), timed over back-to-back calls that rotate over
buffer sets larger than the Infinity Cache; `extras` the rows measured on the step's buffers (W4A4
GEMM, FP4 KV cache, MXFP8, 16x16 tiles).  The CPU oracle is timed on bounded
samples of each workload, on one thread and on every usable core.

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
CONFIG_ROWS = ("tiny_roundtrip", "activations.amax", "activations.nearest_hint", "activations.guided",
               "activations.nearest_hint_from_scratch", "activations.nearest_from_scratch",
               "transpose_requant", "grouped_gemm", "grouped_gemm_w4a4")


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--layers", type=int, default=LAYERS)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="skip the rows measured outside the step (W4A4 GEMM, FP4 KV cache, "
                        "MXFP8, 16x16 tiles)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-configuration rows (tiny round trip, activations, "
                        "8192^2 transpose-requantize, 32-expert grouped GEMM)")
    p.add_argument("--no-step", action="store_true",
                   help="skip the timed MoE-weights step (for profiling the other sections; "
                        "the output line then carries no value)")
    p.add_argument("--reps", type=int, default=20,
                   help="timed calls per configuration row (back to back, rotating over "
                        "buffer sets larger than the Infinity Cache)")
    p.add_argument("--traffic-from", nargs="+", metavar="DIR",
                   help="write profiles/hbm_traffic.json from rocprofv3 counter CSVs under DIR "
                        "(read-request and write-request passes) and exit")
    p.add_argument("--traffic-section", default="step",
                   help="step, or configs/ROW for one configuration row (see --config-row)")
    p.add_argument("--config-row", metavar="ROW",
                   help="run only this configuration row (and its set-up), e.g. for one "
                        "counter pass per row: " + ", ".join(CONFIG_ROWS))
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run one 1 GiB device copy (reference for HBM byte counters)")
    return p.parse_args()


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(traffic_from(args.traffic_from, args.traffic_section)[args.traffic_section]))
        return
    if args.config_row is not None and args.config_row not in CONFIG_ROWS:
        sys.exit(f"--config-row must be one of {', '.join(CONFIG_ROWS)}")
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the path has no "
                                   "multi-GPU leg (--gpus must be 1)"}))
        sys.exit(2)

    import torch

    from fp4_quantization_precision_amd import _lib

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = _lib.lib()
    stream = torch.cuda.current_stream()

    line = {
        "metric": "quantize/guided-quantize GB/s and % of HBM peak; grouped-GEMM TFLOP/s",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
    }
    step = None
    if not args.no_step:
        step = measure_step(args, L, dev, stream)
        line.update(step["line"])
    else:
        line["config"] = {"workload": "per-configuration rows only (no step)"}
    if step is not None:
        line["copy_ceiling"] = copy_ceiling(dev, stream)
        for ent in line["kernels"].values():
            if "GB/s" in ent and "frac_hbm_peak" in ent:
                ent["frac_copy_ceiling"] = round(ent["GB/s"] / line["copy_ceiling"]["GB/s"], 4)
    configs = None if args.no_configs else measure_configs(L, dev, stream, args.reps, args.config_row)
    extras = None
    if step is not None and not args.no_extras:
        extras = measure_extras(L, dev, stream, *step["extras_args"])
    cpu = None
    if step is not None and not args.no_cpu_baseline:
        cpu = cpu_baseline(*step["cpu_args"])
    line["cpu_baseline"] = cpu
    line["configs"] = configs
    line["extras"] = extras
    if args.copy_calibration:
        # one plain device copy of 1 GiB (read 1 GiB, write 1 GiB): a yardstick of
        # known size for the HBM byte counters of the kernels above
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    print(json.dumps(line), flush=True)


def copy_ceiling(dev, stream, reps=10):
    """A measured HBM ceiling: torch's device copy of 1 GiB (1 GiB read, 1 GiB
    written), average of `reps` back-to-back copies timed with events on `stream`;
    the two buffers together exceed the Infinity Cache."""
    import torch
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        us = _time_phase(stream, lambda: dst.copy_(src), reps)
    del src, dst
    moved = 2.0 * (1 << 30)
    return {"kernel": "torch copy_ (device to device)", "bytes_per_copy": moved, "avg_us": round(us, 2),
            "GB/s": round(moved / us / 1e3, 1), "frac_hbm_peak": round(moved / us / 1e3 / HBM_PEAK_GBS, 4)}


def measure_step(args, L, dev, stream):
    """The timed MoE-weights step (all rows of the hot path over the 48-layer
    workload).  Returns the output-line fields and the buffers the extras and the
    CPU baseline reuse."""
    import numpy as np
    import torch

    from fp4_quantization_precision_amd import inputs, ops
    from fp4_quantization_precision_amd._lib import TQ_AMAX_GIVEN, TQ_BF16

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
        ent = {"kernel": KERNEL_OF[cat][0], "launches_per_step": cat_n[cat],
               "layers_per_launch": cat_layers[cat] / cat_n[cat], "avg_us": round(us, 2)}
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

    # the roofline is reported for the kernel with the largest share of the step
    dom_cat = max(kernels, key=lambda c: kernels[c]["share_of_step"])
    dom = kernels[dom_cat]
    if dom_cat == "gemm":
        roofline = {"bound": "mfma", "achieved": dom["TFLOP/s"], "peak": BF16_MFMA_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": dom["frac_bf16_mfma_peak"]}
    else:
        roofline = {"bound": "hbm", "achieved": dom["GB/s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": dom["frac_hbm_peak"]}
    roofline.update({"traffic": measured_traffic(dom_cat, dom["layers_per_launch"]),
                     "kernel": dom["kernel"], "category": dom_cat,
                     "algorithmic_bytes_per_launch": call_bytes(dom_cat),
                     "avg_launch_us": dom["avg_us"], "share_of_step": dom["share_of_step"]})
    if dom_cat == "gemm":
        roofline["algorithmic_flops_per_launch"] = gemm_flops

    fields = {
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "ms_per_step": round(ms_per_step, 3),
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
        "kernels": kernels,
        "mismatch": mism,
        "input_generation_s": round(t_gen, 1),
    }
    return {"line": fields,
            "extras_args": (A, OFF, QG, QN, nl, first_hint),
            "cpu_args": (XR, XT, A, counts, first_hint)}


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


def _time_rotating(stream, call, n_sets, reps):
    """Event times (us) of `reps` back-to-back calls call(i), where call i works on
    buffer set i % n_sets; the sets together exceed the 256 MiB Infinity Cache, so a
    call finds little of its input in cache.  One warm-up pass over the sets first.

    avg_us: one event on the launch stream before the first call and one after the
    last, so the span holds the calls and the dispatch gaps between them only; the
    rates are taken from it.  median_us: a second pass with an event before every
    call, the median of the per-call spans; each of those also holds one event
    record, which costs from under 1 to about 5 us depending on the machine, so it
    is reported for the spread, not rated."""
    import statistics

    import torch
    for i in range(n_sets):
        call(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(reps):
        call(i % n_sets)
    e1.record(stream)
    torch.cuda.synchronize()
    avg = 1e3 * e0.elapsed_time(e1) / reps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    for i in range(reps):
        ev[i].record(stream)
        call(i % n_sets)
    ev[reps].record(stream)
    torch.cuda.synchronize()
    per = [1e3 * ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]
    return {"avg_us": round(avg, 2), "median_us": round(statistics.median(per), 2), "calls": reps,
            "buffer_sets": n_sets}


def _config_traffic(row, kernel):
    """Counter-measured HBM bytes per call of a configuration row (the sum over its
    kernels, from the counter passes of that row run alone), or None if not
    measured on the current sources."""
    if row is None:
        return None
    tot = 0
    for k in kernel.split(" + "):
        ent = _traffic_entry("configs/" + row, k)
        if ent is None:
            return None
        tot += ent["bytes_per_dispatch"]
    return tot


def _bw_row(kernel, timing, alg_bytes, moved_bytes=None, note=None, row=None):
    """A bandwidth-bound configuration row (rates from the back-to-back average); `row`
    names its counter section."""
    us = timing["avg_us"]
    gbs = alg_bytes / us / 1e3
    out = {"kernel": kernel, **timing, "algorithmic_bytes": alg_bytes, "GB/s": round(gbs, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": _config_traffic(row, kernel)}}
    if moved_bytes is not None:
        out["moved_bytes"] = moved_bytes
        out["GB/s_moved"] = round(moved_bytes / us / 1e3, 1)
        out["frac_hbm_peak_moved"] = round(moved_bytes / us / 1e3 / HBM_PEAK_GBS, 4)
    if note:
        out["note"] = note
    return out


def _mfma_row(kernel, timing, flops, note=None, row=None):
    """An MFMA-bound configuration row (rates from the back-to-back average); `row`
    names its counter section."""
    us = timing["avg_us"]
    tf = flops / us / 1e6
    out = {"kernel": kernel, **timing, "flops": flops, "TFLOP/s": round(tf, 1),
           "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                        "traffic": _config_traffic(row, kernel)}}
    if note:
        out["note"] = note
    return out


def measure_configs(L, dev, stream, reps, only=None):
    """One row per workload configuration.  Each row times `reps` back-to-back calls
    with HIP events on the launch stream, rotating over buffer sets that together
    exceed the 256 MiB Infinity Cache; rates come from the average over a span of
    back-to-back calls, and the median of event-bracketed calls is reported beside it:

    * tiny round trip, 64 x 256 fp32: the whole chain (launch-bound; no roofline claim);
    * activations, 32768 x 4096 bf16 (rollout and trainer copies alternate): tensor
      amax; nearest + hint and guided with the tensor amax given; and tq_quantize from
      scratch (amax pass + quantize pass);
    * transpose-requantize of an 8192 x 8192 NVFP4 tensor, one call per seed, over
      five source tensors;
    * grouped GEMM, 32 experts, Zipf(1.1) counts over 16384 tokens, K 2048, N 768,
      over three input sets; and the same with NVFP4 activations.

    `only` names one row (CONFIG_ROWS) to run alone, with its set-up, e.g. for a
    counter pass per row."""
    import torch

    from fp4_quantization_precision_amd import inputs, ops
    from fp4_quantization_precision_amd._lib import TQ_AMAX_GIVEN, TQ_BF16, TQ_F32

    sp = C.c_void_p(stream.cuda_stream)
    P = lambda t: C.c_void_p(t.data_ptr()) if t is not None else None
    out = {}
    want = lambda *rows: only is None or only in rows

    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {L.tq_status_string(st).decode()}")

    # ---- tiny round trip ----
    if want("tiny_roundtrip"):
        xr, xt = (t.to(dev) for t in inputs.tiny_roundtrip())
        n1 = xr.numel()
        h1 = torch.empty(ops.hint_words(n1), dtype=torch.int32, device=dev)
        q1 = [ops.new_nvfp4((1,), 64, 256, dev) for _ in range(3)]
        c1 = torch.empty((2, 2), dtype=torch.int64, device=dev)
        pair = torch.empty((2, 2, n1 // 2), dtype=torch.uint8, device=dev)

        def tiny(_):
            ok(L.tq_quantize(P(xr), TQ_F32, 1, 64, 256, P(q1[0].tensor_amax), P(q1[0].codes),
                             P(q1[0].scales), P(q1[0].tensor_scale), P(h1), 0, sp), "tiny nearest+hint")
            ok(L.tq_quantize(P(xt), TQ_F32, 1, 64, 256, P(q1[1].tensor_amax), P(q1[1].codes),
                             P(q1[1].scales), P(q1[1].tensor_scale), None, 0, sp), "tiny nearest")
            ok(L.tq_quantize_guided(P(xt), TQ_F32, 1, 64, 256, P(q1[2].tensor_amax), P(h1),
                                    P(q1[2].codes), P(q1[2].scales), P(q1[2].tensor_scale), 0, sp),
               "tiny guided")
            ok(L.tq_code_mismatch(P(pair[0]), P(pair[1]), 2, n1, P(c1), sp), "tiny mismatch")
        t1 = _time_rotating(stream, tiny, 1, reps)
        out["tiny_roundtrip"] = {
            "workload": "tiny round trip: 64 x 256 fp32 X_r, X_t = X_r(1+e); nearest + hint, nearest, "
                        "guided, mismatch counts (7 kernels incl. amax passes and fills)",
            **t1, "note": "launch-bound; no roofline claim"}
        del xr, xt, h1, q1, c1, pair

    # ---- activations 32768 x 4096 bf16 ----
    if want("activations.amax", "activations.nearest_hint", "activations.guided",
             "activations.nearest_hint_from_scratch", "activations.nearest_from_scratch"):
        T3, H3 = 32768, 4096
        n3 = T3 * H3
        ar, at, _ = inputs.activations(T3, H3, device=dev)
        X = (ar, at)
        hw = ops.hint_words(n3)
        h3 = [torch.empty(hw, dtype=torch.int32, device=dev) for _ in range(2)]
        qa = [ops.new_nvfp4((1,), T3, H3, dev) for _ in range(2)]
        qs = [ops.new_nvfp4((1,), T3, H3, dev) for _ in range(2)]
        for i in range(2):
            ok(L.tq_tensor_amax(P(X[i]), TQ_BF16, 1, n3, P(qa[i].tensor_amax), sp), "amax")

        def amax(i):
            ok(L.tq_tensor_amax(P(X[i]), TQ_BF16, 1, n3, P(qs[i].tensor_amax), sp), "amax")

        def nearest_hint(i):
            ok(L.tq_quantize(P(X[i]), TQ_BF16, 1, T3, H3, P(qa[i].tensor_amax), P(qa[i].codes),
                             P(qa[i].scales), P(qa[i].tensor_scale), P(h3[i]), TQ_AMAX_GIVEN, sp),
               "nearest+hint")

        def guided(i):
            # the trainer copy guided by the rollout's hints, and (alternating) the reverse
            ok(L.tq_quantize_guided(P(X[1 - i]), TQ_BF16, 1, T3, H3, P(qa[1 - i].tensor_amax), P(h3[i]),
                                    P(qs[i].codes), P(qs[i].scales), P(qs[i].tensor_scale),
                                    TQ_AMAX_GIVEN, sp), "guided")

        def scratch_hint(i):
            ok(L.tq_quantize(P(X[i]), TQ_BF16, 1, T3, H3, P(qs[i].tensor_amax), P(qs[i].codes),
                             P(qs[i].scales), P(qs[i].tensor_scale), P(h3[i]), 0, sp),
               "from-scratch nearest+hint")

        def scratch(i):
            ok(L.tq_quantize(P(X[i]), TQ_BF16, 1, T3, H3, P(qs[i].tensor_amax), P(qs[i].codes),
                             P(qs[i].scales), P(qs[i].tensor_scale), None, 0, sp), "from-scratch nearest")
        b_q, b_h = n3 * (2 + 0.5 + 1 / 16), n3 / 8
        act = {"workload": f"activations [{T3} x {H3}] bf16, Student-t(4), 8 outlier channels x50; "
                           "rollout and trainer copies alternate (268 MiB each)"}
        if want("activations.amax"):
            act["amax"] = _bw_row("tq::amax_kernel<true, 1024>", _time_rotating(stream, amax, 2, reps),
                                  2.0 * n3, row="activations.amax")
        if want("activations.nearest_hint"):
            act["nearest_hint"] = _bw_row("tq::quantize_kernel<true, 1>",
                                          _time_rotating(stream, nearest_hint, 2, reps), b_q + b_h,
                                          note="tensor amax given", row="activations.nearest_hint")
        if want("activations.guided"):
            for i in range(2):  # the hints it reads
                nearest_hint(i)
            act["guided"] = _bw_row("tq::quantize_kernel<true, 2>", _time_rotating(stream, guided, 2, reps),
                                    b_q + b_h, note="hints of the other copy, tensor amax given",
                                    row="activations.guided")
        if want("activations.nearest_hint_from_scratch"):
            act["nearest_hint_from_scratch"] = _bw_row(
                "tq::amax_kernel<true, 1024> + tq::quantize_kernel<true, 1>",
                _time_rotating(stream, scratch_hint, 2, reps), b_q + b_h, b_q + b_h + 2.0 * n3,
                note="tq_quantize without a given amax: fill, amax pass, quantize pass",
                row="activations.nearest_hint_from_scratch")
        if want("activations.nearest_from_scratch"):
            act["nearest_from_scratch"] = _bw_row(
                "tq::amax_kernel<true, 1024> + tq::quantize_kernel<true, 0>",
                _time_rotating(stream, scratch, 2, reps), b_q, b_q + 2.0 * n3,
                note="tq_quantize without a given amax: fill, amax pass, quantize pass",
                row="activations.nearest_from_scratch")
        out["activations"] = act
        del ar, at, X, h3, qa, qs

    # ---- transpose-requantize 8192 x 8192, one call per seed, five source tensors ----
    if want("transpose_requant"):
        R4 = C4_ = 8192
        n4 = R4 * C4_
        srcs = []
        for j in range(5):
            src = inputs.transpose_source(R4, C4_, device=dev, seed=4 if j == 0 else 40 + j)
            srcs.append((ops.quantize(src), ops.new_nvfp4((1,), C4_, R4, dev)))
            del src

        def sr(i):
            q, qt = srcs[i % 5]
            ok(L.tq_requant_transpose_sr(P(q.codes), P(q.scales), P(q.tensor_scale), 1, R4, C4_,
                                         C.c_uint64(i), P(qt.codes), P(qt.scales), P(qt.tensor_scale),
                                         sp), "SR transpose")
        seeds = {"n": 0}

        def sr_seeded(j):  # a new seed for every call
            sr(j + 5 * seeds["n"])
            seeds["n"] += j == 4
        out["transpose_requant"] = {
            "workload": f"NVFP4 [{R4} x {C4_}] (nearest-quantized N(0,1) bf16) -> transposed, "
                        "stochastic-rounding requantize; a new Philox seed per call",
            **_bw_row("tq::requant_transpose_sr_kernel<false>", _time_rotating(stream, sr_seeded, 5, reps),
                      n4 * 2 * (0.5 + 1 / 16), row="transpose_requant")}
        del srcs

    # ---- grouped GEMM: 32 experts, 16384 tokens, K 2048, N 768, three input sets ----
    if want("grouped_gemm", "grouped_gemm_w4a4"):
        G5, T5, K5, N5 = 32, 16384, 2048, 768
        sets = []
        for j in range(3):
            a5, w5, off5 = inputs.grouped_gemm_inputs(G5, T5, K5, N5, device=dev, seed=5 if j == 0 else 50 + j)
            sets.append((a5, off5.to(dev), ops.quantize(w5), ops.quantize(a5.view(1, T5, K5)),
                         torch.empty((T5, N5), dtype=torch.bfloat16, device=dev)))
            del w5

        def gemm(i):
            a5, off5, q5, _, o5 = sets[i]
            ok(L.tq_grouped_gemm_nvfp4(P(a5), P(off5), G5, T5, N5, K5, P(q5.codes), P(q5.scales),
                                       P(q5.tensor_scale), P(o5), sp), "grouped GEMM")

        def w4a4(i):
            _, off5, q5, a5q, o5 = sets[i]
            ok(L.tq_grouped_gemm_w4a4(P(a5q.codes), P(a5q.scales), P(a5q.tensor_scale), P(off5), G5, T5,
                                      N5, K5, P(q5.codes), P(q5.scales), P(q5.tensor_scale), P(o5), sp),
               "W4A4 grouped GEMM")
        flops5 = 2.0 * T5 * K5 * N5
        if want("grouped_gemm"):
            out["grouped_gemm"] = {
                "workload": f"{G5} experts, Zipf(1.1) counts over {T5} tokens, K {K5}, N {N5}; "
                            "A bf16 N(0,1), W NVFP4 from N(0,0.02)",
                **_mfma_row("tq::grouped_gemm_nvfp4_kernel<false, true>",
                            _time_rotating(stream, gemm, 3, reps), flops5, row="grouped_gemm")}
        if want("grouped_gemm_w4a4"):
            out["grouped_gemm_w4a4"] = {
                "workload": "as grouped_gemm, activations NVFP4 (one tensor)",
                **_mfma_row("tq::grouped_gemm_nvfp4_kernel<true, true>",
                            _time_rotating(stream, w4a4, 3, reps), flops5, row="grouped_gemm_w4a4")}
        del sets
    torch.cuda.synchronize()
    return out


def measure_extras(L, dev, stream, A, OFF, QG, QN, nl, first_hint):
    """Rows measured outside the step, on the same device buffers:
    * W4A4 grouped GEMM: each layer's activations quantized to NVFP4 (one tensor),
      then the GEMM with the trainer's NVFP4 weights;
    * FP4 KV cache with hints: one layer's K and V cache [32768 x 8 x 128] bf16,
      rollout nearest + hints and trainer guided, per token-head blocks of 16;
    * 16x16-tile scaling: quantize and exact transpose of the activations
      workload [32768 x 4096] bf16, and the share of zero codes against block-16;
    * MXFP8 for the backward: nearest quantize of the activations workload and the
      NVFP4 -> MXFP8 stochastic-rounding transpose of each layer's trainer weights."""
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
        "kernel": "tq::amax_kernel<true, 1024> + tq::quantize_kernel<true, 0> (tq_quantize from scratch)",
        "avg_us": round(us_q, 2), "GB/s": round(n_a * (2 + 0.5625) / us_q / 1e3, 1),
        "frac_hbm_peak": round(n_a * (2 + 0.5625) / us_q / 1e3 / HBM_PEAK_GBS, 4),
        "GB/s_moved": round(n_a * (4 + 0.5625) / us_q / 1e3, 1),
        "note": "[16384 x 768] bf16 per layer, tensor amax not given: fill, amax pass, quantize "
                "pass; GB/s counts each byte once, GB/s_moved counts the input twice"}
    out["w4a4_gemm"] = {
        "kernel": "tq::grouped_gemm_nvfp4_kernel<true>", "avg_us": round(us_g, 2),
        "TFLOP/s": round(flops / us_g / 1e6, 1),
        "frac_bf16_mfma_peak": round(flops / us_g / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4),
        "shape": f"{EXPERTS} experts, {TOKENS} tokens, K {COLS}, N {ROWS}"}
    del AQ, OUT

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
        "kernel": "tq::amax_kernel<true, 1024> + tq::quantize_kernel<true, 1>", "avg_us": round(us_h, 2),
        "GB/s": round(n * (2 + 0.6875) / us_h / 1e3, 1),
        "frac_hbm_peak": round(n * (2 + 0.6875) / us_h / 1e3 / HBM_PEAK_GBS, 4),
        "GB/s_moved": round(n * (4 + 0.6875) / us_h / 1e3, 1),
        "note": "per K or V tensor [32768 x 8 x 128], tensor amax not given: fill, amax pass, "
                "nearest + hints pass; GB/s counts each byte once, GB/s_moved counts the input twice"}
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
    "amax": ("tq::amax_kernel<true, 256>", "tq_quantize.hip"),
    "quantize": ("tq::quantize_kernel<true, 0>", "tq_quantize.hip"),
    "quantize_hint": ("tq::quantize_kernel<true, 1>", "tq_quantize.hip"),
    "guided": ("tq::quantize_kernel<true, 2>", "tq_quantize.hip"),
    "mismatch": ("tq::mismatch_kernel", "tq_quantize.hip"),
    "sr_transpose": ("tq::requant_transpose_sr_kernel<false>", "tq_sr.hip"),
    "gemm": ("tq::grouped_gemm_nvfp4_kernel<false, true>", "tq_gemm.hip"),
}

# HBM-side traffic.  Two rocprofv3 --pmc passes over this benchmark count the L2's
# requests to the memory fabric per dispatch: TCC_EA0_RDREQ (of which
# TCC_EA0_RDREQ_32B are 32-byte reads; the rest are 128-byte reads on this GPU)
# and TCC_EA0_WRREQ (of which TCC_EA0_WRREQ_64B are 64-byte writes; the rest 32-byte).
# `--traffic-from DIR... --traffic-section step|configs` turns the counter CSVs into
# profiles/hbm_traffic.json, keyed by the SHA-256 of the library's sources, so a
# figure is reported only for the code it was measured on.
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# layers each step kernel covers per step (48 layers, hints for the latter 24)
STEP_LAYERS = {"amax": 96, "quantize": 72, "quantize_hint": 24, "guided": 24, "mismatch": 72,
               "sr_transpose": 48, "gemm": 48}


def _sources_digest():
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "fp4_quantization_precision_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        with open(os.path.join(d, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _short_kernel(name):
    import re
    name = name.replace("void ", "", 1)
    m = re.match(r"([\w:]+(<[^()]*>)?)", name)
    return m.group(1) if m else name


def traffic_from(dirs, section):
    """Per-kernel HBM bytes from rocprofv3 counter CSVs (one --pmc pass with the read
    request counters, one with the write request counters) into TRAFFIC_JSON."""
    import csv
    import glob
    per = {}  # kernel -> {counter: {dispatch: value}}
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = _short_kernel(r["Kernel_Name"])
                    c = r["Counter_Name"].replace("_sum", "")
                    per.setdefault(k, {}).setdefault(c, {})[r["Dispatch_Id"]] = float(r["Counter_Value"])
    kernels = {}
    for k, cs in per.items():
        if not k.startswith("tq::"):  # input generation and other library kernels
            continue
        need = ("TCC_EA0_RDREQ", "TCC_EA0_RDREQ_32B", "TCC_EA0_WRREQ", "TCC_EA0_WRREQ_64B")
        if not all(c in cs for c in need):
            continue
        tot = {c: sum(cs[c].values()) for c in need}
        n = len(cs["TCC_EA0_RDREQ"])
        rd = 128 * (tot["TCC_EA0_RDREQ"] - tot["TCC_EA0_RDREQ_32B"]) + 32 * tot["TCC_EA0_RDREQ_32B"]
        wr = 64 * tot["TCC_EA0_WRREQ_64B"] + 32 * (tot["TCC_EA0_WRREQ"] - tot["TCC_EA0_WRREQ_64B"])
        ent = {"dispatches": n, "read_bytes_per_dispatch": round(rd / n),
               "write_bytes_per_dispatch": round(wr / n), "bytes_per_dispatch": round((rd + wr) / n),
               "counters_per_dispatch": {c: round(v / n, 1) for c, v in tot.items()}}
        kernels[k] = ent
    if section == "step":
        for cat, (kname, _) in KERNEL_OF.items():
            if kname in kernels:
                e = kernels[kname]
                e["bytes_per_layer"] = round(e["bytes_per_dispatch"] * e["dispatches"] / STEP_LAYERS[cat])
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        with open(TRAFFIC_JSON) as fh:
            data = json.load(fh)
    data[section] = {"sources_sha256": _sources_digest(), "kernels": kernels}
    data["method"] = ("bytes = 128 x (TCC_EA0_RDREQ - TCC_EA0_RDREQ_32B) + 32 x TCC_EA0_RDREQ_32B "
                      "+ 64 x TCC_EA0_WRREQ_64B + 32 x (TCC_EA0_WRREQ - TCC_EA0_WRREQ_64B), "
                      "summed over the XCDs' L2 channels, averaged per dispatch")
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    return data


def _traffic_entry(section, kname):
    if not os.path.exists(TRAFFIC_JSON):
        return None
    with open(TRAFFIC_JSON) as fh:
        sec = json.load(fh).get(section)
    if not sec or sec.get("sources_sha256") != _sources_digest():
        return None
    return sec["kernels"].get(kname)


def measured_traffic(cat, layers_per_launch):
    """Counter-measured HBM bytes per launch of a step kernel, or None if not measured
    on the current sources."""
    ent = _traffic_entry("step", KERNEL_OF[cat][0])
    if ent is None or "bytes_per_layer" not in ent:
        return None
    return round(ent["bytes_per_layer"] * layers_per_launch)


def _cpu_threads():
    """Host threads for the threaded oracle runs: every core this process may use,
    at most 16 (the host share of one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def _run_units(unit, n_units, threads):
    """Wall time of unit(0..n_units-1) on `threads` host threads (the oracle's C
    calls release the GIL, so the threads run in parallel)."""
    from concurrent.futures import ThreadPoolExecutor
    t0 = time.perf_counter()
    if threads == 1:
        for i in range(n_units):
            unit(i)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(unit, range(n_units)))
    return time.perf_counter() - t0


def cpu_baseline(XR, XT, A, counts, first_hint):
    """The CPU oracle as it stands, timed on the host on bounded samples of each
    workload, once on one thread and once on every usable core (one sample unit per
    thread; the oracle's C routines release the GIL).  Rates use the same
    algorithmic bytes (or flops) as the GPU rows.

    * step: per unit, one expert of layer `first_hint` (a hinted layer) through
      amax (both copies), nearest + hint, nearest, guided, two mismatch counts and
      the SR transpose, plus that expert's share of the layer's grouped GEMM (256 of
      16384 token rows, fp64);
    * activations: per unit, 1024 rows x 4096: amax, nearest + hint, guided;
    * transpose-requantize: per unit, a 1024-row slab of the 8192^2 NVFP4 tensor;
    * grouped GEMM 32 experts, K 2048, N 768: per unit, 64 token rows in fp64."""
    import numpy as np
    import torch

    import oracle
    from fp4_quantization_precision_amd import inputs

    T = _cpu_threads()
    res = {}

    def rates(name, unit, unit_bytes=None, unit_flops=None, what=""):
        t1 = _run_units(unit, 1, 1)
        tT = _run_units(unit, T, T)
        r = {"sample_unit": what, "units_all_cores": T, "seconds_1core": round(t1, 3),
             "seconds_all_cores": round(tT, 3)}
        if unit_bytes is not None:
            r["GB/s_1core"] = round(unit_bytes / t1 / 1e9, 5)
            r["GB/s_all_cores"] = round(T * unit_bytes / tT / 1e9, 5)
        if unit_flops is not None:
            r["GFLOP/s_1core"] = round(unit_flops / t1 / 1e9, 4)
            r["GFLOP/s_all_cores"] = round(T * unit_flops / tT / 1e9, 4)
        res[name] = r
        return r

    # ---- step sample (MoE weights, one hinted layer) ----
    l, per = first_hint, ROWS * COLS
    xr_l = XR[l].cpu()
    xt_l = XT[l].cpu()
    a_l = A[l].cpu()
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    # untimed: the layer's trainer weights in the oracle's own encoding for the GEMM rows
    wq_parts = [None] * EXPERTS

    def prep(e):
        wq_parts[e] = oracle.quantize(xt_l[e], 1, ROWS, COLS)
    _run_units(prep, EXPERTS, T)
    wq = {"codes": np.concatenate([q["codes"] for q in wq_parts]),
          "scales": np.concatenate([q["scales"] for q in wq_parts]),
          "tensor_scale": np.concatenate([q["tensor_scale"] for q in wq_parts])}
    del wq_parts

    def step_unit(i):
        e = i % EXPERTS
        xr, xt = xr_l[e], xt_l[e]
        oracle.tensor_amax(xr, 1, per)
        am = oracle.tensor_amax(xt, 1, per)
        qr = oracle.quantize(xr, 1, ROWS, COLS)
        h = oracle.extract_hint(qr["codes"], per)
        qn = oracle.quantize(xt, 1, ROWS, COLS, amax=am)
        qg = oracle.quantize_guided(xt, 1, ROWS, COLS, h, amax=am)
        oracle.code_mismatch(qr["codes"], qn["codes"], 1, per)
        oracle.code_mismatch(qr["codes"], qg["codes"], 1, per)
        oracle.requant_transpose_sr(qg["codes"], qg["scales"], qg["tensor_scale"], 1, ROWS, COLS, 1)
        rows = np.arange(e, TOKENS, EXPERTS)  # 256 rows spread over the layer
        oracle.grouped_gemm(a_l, off, ROWS, COLS, wq["codes"], wq["scales"], wq["tensor_scale"],
                            rows=rows)
    chain_b = per * (2.0 * 2 + (2 + 0.5 + 1 / 16 + 1 / 8) + (2 + 0.5 + 1 / 16) +
                     (2 + 1 / 8 + 0.5 + 1 / 16) + 2 * 1.0 + 2 * (0.5 + 1 / 16))
    gemm_b = (TOKENS * COLS * 2 + EXPERTS * per * (0.5 + 1 / 16) + TOKENS * ROWS * 2) / EXPERTS
    step = rates("step", step_unit, unit_bytes=chain_b + gemm_b,
                 what=f"one expert of layer {l} ({per} weights) through the step's quantizer chain "
                      f"and SR transpose, plus {TOKENS // EXPERTS} fp64 grouped-GEMM rows")
    del xr_l, xt_l, a_l, wq

    # ---- activations ----
    T3, H3, R3 = 32768, 4096, 1024
    ar, at, _ = inputs.activations(T3, H3, device=XR.device)
    ar_h, at_h = ar.cpu(), at.cpu()
    del ar, at
    # the whole tensor's maxima, given to the sampled rows (untimed)
    am_r = float(oracle.tensor_amax(ar_h, 1, T3 * H3)[0])
    am_t = float(oracle.tensor_amax(at_h, 1, T3 * H3)[0])
    ar_c, at_c = ar_h[: R3 * T], at_h[: R3 * T]
    del ar_h, at_h

    def act_unit(i):
        xr, xt = ar_c[i * R3:(i + 1) * R3], at_c[i * R3:(i + 1) * R3]
        oracle.tensor_amax(xr, 1, R3 * H3)
        q = oracle.quantize(xr, 1, R3, H3, amax=[am_r])
        h = oracle.extract_hint(q["codes"], R3 * H3)
        oracle.quantize_guided(xt, 1, R3, H3, h, amax=[am_t])
    rates("activations", act_unit, unit_bytes=R3 * H3 * (2 + 2 * (2.5625 + 0.125)),
          what=f"{R3} rows x {H3}: amax, nearest + hint, guided")
    del ar_c, at_c

    # ---- transpose-requantize slabs of the 8192^2 tensor ----
    R4, C4_ = 1024, 8192
    n_slabs = min(T, 8192 // R4)  # more threads than slabs reuse them
    src = inputs.transpose_source(8192, 8192, device=XR.device)[: R4 * n_slabs].cpu()
    slabs = [None] * n_slabs

    def prep4(i):
        slabs[i] = oracle.quantize(src[i * R4:(i + 1) * R4], 1, R4, C4_)
    _run_units(prep4, n_slabs, T)

    def sr_unit(i):
        q = slabs[i % n_slabs]
        oracle.requant_transpose_sr(q["codes"], q["scales"], q["tensor_scale"], 1, R4, C4_, i)
    rates("transpose_requant", sr_unit, unit_bytes=R4 * C4_ * 2 * (0.5 + 1 / 16),
          what=f"a {R4} x {C4_} slab of the nearest-quantized 8192^2 tensor")
    del src, slabs

    # ---- grouped GEMM rows, 32 experts ----
    G5, T5, K5, N5, R5 = 32, 16384, 2048, 768, 64
    a5, w5, off5 = inputs.grouped_gemm_inputs(G5, T5, K5, N5, device=XR.device, seed=5)
    a5, w5 = a5.cpu(), w5.cpu()
    parts = [None] * G5

    def prep5(e):
        parts[e] = oracle.quantize(w5[e], 1, N5, K5)
    _run_units(prep5, G5, T)
    w5q = {k: np.concatenate([q[k] for q in parts]) for k in ("codes", "scales", "tensor_scale")}
    del parts, w5

    def gemm_unit(i):
        rows = np.arange(i, T5, T5 // R5)[:R5]
        oracle.grouped_gemm(a5, off5, N5, K5, w5q["codes"], w5q["scales"], w5q["tensor_scale"],
                            rows=rows)
    rates("grouped_gemm", gemm_unit, unit_flops=2.0 * R5 * K5 * N5,
          what=f"{R5} token rows spread over the {G5} experts, fp64")

    return {"value": step["GB/s_all_cores"], "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": f"per thread: {step['sample_unit']}; {T} threads, "
                      f"{step['seconds_all_cores']} s",
            "value_1core": step["GB/s_1core"], "per_config": res}


if __name__ == "__main__":
    main()

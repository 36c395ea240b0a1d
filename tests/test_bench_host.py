"""Host-side logic of bench.py (CPU only): the HBM byte count from the L2's
memory-request counters, the per-section traffic table keyed by the sources'
digest, kernel-name shortening, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import bench

FIELDS = ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"]


def _write_counters(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_short_kernel_names():
    assert bench._short_kernel("void tq::quantize_kernel<true, 1>(void const*, long)") == \
        "tq::quantize_kernel<true, 1>"
    assert bench._short_kernel("tq::mismatch_kernel(HIP_vector_type<unsigned int, 4u> const*)") == \
        "tq::mismatch_kernel"


def test_traffic_from_request_counts(tmp_path, monkeypatch):
    """Two dispatches of one kernel: reads are 128-byte requests except the 32-byte
    ones, writes 64-byte requests except the 32-byte ones; averages per dispatch,
    library kernels only, per-layer bytes for the step section."""
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    k = "void tq::amax_kernel<true, 256>(HIP_vector_type<unsigned int, 4u> const*, long, long, float*)"
    other = "void at::native::vectorized_elementwise_kernel<4>(int)"
    rd = [(k, "TCC_EA0_RDREQ_sum", 1, 1000), (k, "TCC_EA0_RDREQ_32B_sum", 1, 200),
          (k, "TCC_EA0_RDREQ_sum", 2, 3000), (k, "TCC_EA0_RDREQ_32B_sum", 2, 0),
          (other, "TCC_EA0_RDREQ_sum", 3, 5), (other, "TCC_EA0_RDREQ_32B_sum", 3, 0)]
    wr = [(k, "TCC_EA0_WRREQ_sum", 1, 10), (k, "TCC_EA0_WRREQ_64B_sum", 1, 4),
          (k, "TCC_EA0_WRREQ_sum", 2, 30), (k, "TCC_EA0_WRREQ_64B_sum", 2, 30),
          (other, "TCC_EA0_WRREQ_sum", 3, 1), (other, "TCC_EA0_WRREQ_64B_sum", 3, 1)]
    _write_counters(str(tmp_path / "rd" / "x" / "rd_counter_collection.csv"), rd)
    _write_counters(str(tmp_path / "wr" / "wr_counter_collection.csv"), wr)
    data = bench.traffic_from([str(tmp_path / "rd"), str(tmp_path / "wr")], "step")
    assert data["step"]["sources_sha256"] == bench._sources_digest()
    kernels = data["step"]["kernels"]
    assert list(kernels) == ["tq::amax_kernel<true, 256>"]
    e = kernels["tq::amax_kernel<true, 256>"]
    read = 128 * (4000 - 200) + 32 * 200
    write = 64 * 34 + 32 * (40 - 34)
    assert e["dispatches"] == 2
    assert e["read_bytes_per_dispatch"] == round(read / 2)
    assert e["write_bytes_per_dispatch"] == round(write / 2)
    assert e["bytes_per_dispatch"] == round((read + write) / 2)
    # the step's amax covers 96 layers per step over its two dispatches
    assert e["bytes_per_layer"] == round(e["bytes_per_dispatch"] * 2 / bench.STEP_LAYERS["amax"])
    # read back through the table, and null once the digest no longer matches
    assert bench.measured_traffic("amax", 48) == round(e["bytes_per_layer"] * 48)
    with open(bench.TRAFFIC_JSON) as fh:
        stored = json.load(fh)
    stored["step"]["sources_sha256"] = "0" * 64
    with open(bench.TRAFFIC_JSON, "w") as fh:
        json.dump(stored, fh)
    assert bench.measured_traffic("amax", 48) is None


def test_config_row_traffic_sums_kernels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(tmp_path / "traffic.json"))
    sec = {"sources_sha256": bench._sources_digest(), "kernels": {
        "tq::amax_kernel<true, 1024>": {"bytes_per_dispatch": 100},
        "tq::quantize_kernel<true, 0>": {"bytes_per_dispatch": 250}}}
    with open(bench.TRAFFIC_JSON, "w") as fh:
        json.dump({"configs/activations.nearest_from_scratch": sec}, fh)
    k = "tq::amax_kernel<true, 1024> + tq::quantize_kernel<true, 0>"
    assert bench._config_traffic("activations.nearest_from_scratch", k) == 350
    assert bench._config_traffic("activations.amax", k) is None
    assert bench._config_traffic(None, k) is None


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]

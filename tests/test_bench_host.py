"""Host-side logic of bench.py, on the CPU: the refusal of more than one GPU,
the traffic record's copy calibration (each counter scaled by what it reads
for a 1 GiB device copy, the diagnostic instantiation left out) and the gate
that reports the record only while the kernel sources hash as they did."""

import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

REGULAR = "void flamia::attn_bwd8_kernel<128, false, false, false, true, false, false>(flamia::BwdArgs)"
DIAG = "void flamia::attn_bwd8_kernel<128, false, false, false, true, true, false>(flamia::BwdArgs)"
COPY = "__amd_rocclr_copyBuffer"


def _counter_csv(run_dir, counter, rows):
    os.makedirs(run_dir)
    with open(os.path.join(run_dir, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stdout + r.stderr


def test_diag_instantiation_is_recognised():
    assert bench.is_diag_instantiation(DIAG)
    assert not bench.is_diag_instantiation(REGULAR)
    assert not bench.is_diag_instantiation("void flamia::attn_fwd_kernel<128, 0, false, true, true, false, false>(x)")


def test_traffic_record_is_copy_calibrated_and_gated(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda path: "sources-a")
    (tmp_path / "profiles").mkdir()
    fetch, write = str(tmp_path / "fetch"), str(tmp_path / "write")
    # the 1 GiB copy reads as half its bytes (FETCH) and as all of them (WRITE)
    _counter_csv(fetch, "FETCH_SIZE", [(COPY, 524288.0), (REGULAR, 100.0), (REGULAR, 300.0), (DIAG, 1e6)])
    _counter_csv(write, "WRITE_SIZE", [(COPY, 1048576.0), (REGULAR, 50.0), (DIAG, 1e6)])
    bench.write_traffic(fetch, write, 3, "the command", "attn_bwd8_kernel")
    with open(tmp_path / "profiles" / "attn_bwd8_kernel_config3_traffic.json") as f:
        rec = json.load(f)
    assert rec["FETCH_SIZE"]["dispatches"] == 2 and rec["WRITE_SIZE"]["dispatches"] == 1
    assert rec["FETCH_SIZE"]["scale"] == 2.0 and rec["WRITE_SIZE"]["scale"] == 1.0
    assert rec["FETCH_SIZE"]["bytes_per_launch"] == 200.0 * 1024 * 2
    assert rec["WRITE_SIZE"]["bytes_per_launch"] == 50.0 * 1024
    assert rec["hbm_bytes_per_launch"] == 200.0 * 1024 * 2 + 50.0 * 1024
    assert rec["source_sha"] == "sources-a" and rec["command"] == "the command"
    # reported while the sources hash as they did, null once they change
    assert bench.measured_traffic("attn_bwd8_kernel", "config3") == rec["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "source_hash", lambda path: "sources-b")
    assert bench.measured_traffic("attn_bwd8_kernel", "config3") is None
    assert bench.measured_traffic("attn_bwd8_kernel", "config9") is None


def test_weighted_peak_of_the_backward_mix():
    # backward: 8 d N_p at the FP8 peak and 2 d N_p at the bf16 peak
    _, bwd = bench.product_mix(128, 1000, mixed=False)
    assert sum(f for f, _ in bwd) == 10 * 128 * 1000
    peak = bench.weighted_peak(bwd)
    assert abs(peak - 10 / (8 / bench.FP8_PEAK_TFLOPS + 2 / bench.BF16_PEAK_TFLOPS)) < 1e-9

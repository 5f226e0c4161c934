"""bench.py's host-side logic on the CPU: the one-GPU contract, traffic recording and its source-hash guard,
and the algorithmic byte count the roofline line reports."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr and not r.stdout


def test_algorithmic_bytes_of_the_130m_layer():
    """x, delta, z read and y written (bf16), B and C read, A, Dskip, dt_bias read, h_L written (fp32)."""
    batch, L, D, N = 8, 2048, 1536, 16
    assert bench.algorithmic_bytes(batch, L, D) == (4 * batch * L * D * 2 + 2 * batch * L * N * 2 + D * 18 * 4
                                                     + batch * D * N * 4) == 203272192


def _counter_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n")
        for i, (kernel, value) in enumerate(rows):
            f.write(f'{i},"{kernel}",{counter},{value}\n')
    return str(path)


def test_record_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """FETCH_SIZE that reads half of the 256 MiB copy gets factor 2, WRITE_SIZE that reads it exactly factor
    1; a kernel's bytes per launch are the per-dispatch averages scaled by them, and the record is tied to
    the hash of the kernel sources."""
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    kib = bench.CALIB_BYTES / 1024
    cal_f = _counter_csv(tmp_path / "cf.csv", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", kib / 2)] * 3)
    cal_w = _counter_csv(tmp_path / "cw.csv", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib)] * 3)
    fetch = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("void s6_chunk_out<...>(S6Args)", 100.0),
                                                            ("void s6_chunk_out<...>(S6Args)", 300.0),
                                                            ("void s6_chunk_carry<...>(S6Args)", 50.0)])
    write = _counter_csv(tmp_path / "w.csv", "WRITE_SIZE", [("void s6_chunk_out<...>(S6Args)", 40.0),
                                                            ("void s6_chunk_out<...>(S6Args)", 40.0),
                                                            ("void s6_chunk_carry<...>(S6Args)", 10.0)])
    bench.record_traffic("mamba-130m-layer", fetch, write, cal_f, cal_w)
    t = json.load(open(tmp_path / "traffic.json"))
    assert t["_calibration"]["fetch_factor"] == 2.0 and t["_calibration"]["write_factor"] == 1.0
    out = t["mamba-130m-layer"]["s6_chunk_out"]
    assert out["bytes_per_launch"] == (200.0 * 2 + 40.0) * 1024
    assert t["mamba-130m-layer"]["s6_chunk_carry"]["bytes_per_launch"] == (50.0 * 2 + 10.0) * 1024
    assert "s6_step" not in t["mamba-130m-layer"]          # no rows: not recorded
    assert bench.measured_traffic("mamba-130m-layer", "s6_chunk_out") == out["bytes_per_launch"]
    # kernel sources changed since the counters were taken: no traffic figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda workload="": "0" * 16)
    assert bench.measured_traffic("mamba-130m-layer", "s6_chunk_out") is None


def test_kernel_names_match_whole_words_only(tmp_path):
    """s6_carry_scan must not pick up s6_carry_scan2's rows."""
    p = _counter_csv(tmp_path / "f.csv", "FETCH_SIZE", [("void s6_carry_scan2(S6FoldArgs)", 7.0),
                                                        ("void s6_carry_scan(S6FoldArgs)", 3.0)])
    assert bench._pmc(p, "FETCH_SIZE", "s6_carry_scan") == 3.0
    assert bench._pmc(p, "FETCH_SIZE", "s6_carry_scan2") == 7.0
    with pytest.raises(SystemExit):
        bench._pmc(p, "FETCH_SIZE", "s6_step")


"""bench.py on the host: the one-GPU contract, the counter calibration that
turns rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes, the trace summary, and
that a traffic figure is only reported while the kernel sources it was
measured on are unchanged (CPU only)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_from_counters_scaling():
    # the 1 GiB copy reads as 512 MiB through FETCH_SIZE (scale 2) and 1 GiB through WRITE_SIZE (scale 1)
    means = {("__amd_rocclr_copyBuffer", "FETCH_SIZE"): 524288.0,
             ("__amd_rocclr_copyBuffer", "WRITE_SIZE"): 1048576.0,
             ("v_absmax_kernel<128>", "FETCH_SIZE"): 50.0,
             ("v_absmax_kernel<128>", "WRITE_SIZE"): 1.0,
             ("vt_dense_kernel<128>", "FETCH_SIZE"): 100.0,
             ("vt_dense_kernel<128>", "WRITE_SIZE"): 200.0,
             ("mmdit::attn_bf16_kernel<128, 1, 8>", "FETCH_SIZE"): 1000.0,
             ("mmdit::attn_bf16_kernel<128, 1, 8>", "WRITE_SIZE"): 300.0}
    t = bench.traffic_from_counters(means)
    assert t["fetch_scale"] == 2.0 and t["write_scale"] == 1.0
    assert t["kernels"]["vt_dense_kernel"] == {"fetch_bytes": 200 * 1024, "write_bytes": 200 * 1024}
    assert t["kernels"]["attn_bf16_kernel"] == {"fetch_bytes": 2000 * 1024, "write_bytes": 300 * 1024}
    assert t["kernels"]["v_absmax_kernel"] == {"fetch_bytes": 100 * 1024, "write_bytes": 1 * 1024}
    assert t["bytes_per_launch"] == (100 + 1 + 200 + 200 + 2000 + 300) * 1024
    assert t["source_sha256"] == bench.kernel_source_hash()
    del means[("vt_dense_kernel<128>", "WRITE_SIZE")]
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(means)


def test_measured_traffic_follows_source_hash(monkeypatch, tmp_path):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic() is None                      # no file
    path.write_text(json.dumps({"bytes_per_launch": 123, "source_sha256": bench.kernel_source_hash()}))
    assert bench.measured_traffic() == 123
    path.write_text(json.dumps({"bytes_per_launch": 123, "source_sha256": "0" * 64}))
    assert bench.measured_traffic() is None                      # kernel changed since


def test_summarize_kernel_trace(tmp_path, capsys):
    path = tmp_path / "trace_kernel_trace.csv"
    rows = [("void mmdit::attn_bf16_kernel<128, 1, 8>(mmdit::AttnArgs)", 1683456, 512, 0, 13_000_000),
            ("void mmdit::attn_bf16_kernel<128, 1, 8>(mmdit::AttnArgs)", 1683456, 512, 20_000_000, 34_000_000),
            ("mmdit::rope_kernel<8>(mmdit::RopeArgs)", 13262592, 256, 40_000_000, 40_170_000)]
    with open(path, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Grid_Size_X", "Workgroup_Size_X", "Start_Timestamp", "End_Timestamp"])
        wr.writerows(rows)
    bench.summarize([str(path)])
    out = capsys.readouterr().out
    line = [l for l in out.splitlines() if "attn_bf16_kernel" in l][0]
    cells = [c.strip() for c in line.split("|")]
    assert cells[2:8] == ["1683456", "512", "2", "13.500", "13.000", "14.000"]
    assert any("rope_kernel" in l and "0.170" in l for l in out.splitlines())


def test_parse_smi_metrics():
    # shape of `amd-smi metric -c -p --json` (one GPU, two of its XCD clocks shown)
    doc = [{"gpu": 0,
            "power": {"socket_power": {"value": 1350, "unit": "W"}, "gfx_voltage": "N/A"},
            "clock": {"gfx_0": {"clk": {"value": 1800, "unit": "MHz"}, "min_clk": {"value": 500, "unit": "MHz"},
                                "max_clk": {"value": 2400, "unit": "MHz"}},
                      "gfx_1": {"clk": {"value": 1900, "unit": "MHz"}, "max_clk": {"value": 2400, "unit": "MHz"}},
                      "mem_0": {"clk": {"value": 2000, "unit": "MHz"}}}}]
    assert bench.parse_smi_metrics(json.dumps(doc)) == (1850.0, 1350.0)
    assert bench.parse_smi_metrics("not json") == (None, None)
    assert bench.parse_smi_metrics(json.dumps([{"gpu": 0}])) == (None, None)


def test_clock_under_without_amd_smi(monkeypatch):
    import shutil
    monkeypatch.setattr(shutil, "which", lambda name: None)
    calls = []
    assert bench.clock_under(None, lambda: calls.append(1)) is None
    assert calls == []          # nothing is run when there is no tool to sample with

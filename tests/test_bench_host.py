"""Host-side logic of bench.py (no GPU): the source hash that stamps counter data, the HBM
traffic derived from two counter runs and a calibration copy, the counter summaries, and the
refusal of multi-GPU runs."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture
def fake_root(tmp_path, monkeypatch):
    """A copy of the kernel sources under a temporary root that bench reads instead."""
    src = os.path.join(ROOT, "int4_group_quantized_w4a16_amd", "csrc")
    dst = tmp_path / "int4_group_quantized_w4a16_amd" / "csrc"
    shutil.copytree(src, dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "profiles" / "traffic.json"))
    return dst


def test_source_hash_ignores_comments_and_blank_space_only(fake_root):
    base = bench.kernel_source_hash("qkv_decode.hip")
    path = fake_root / "qkv_decode.hip"
    text = path.read_text()
    path.write_text("// a new comment line\n" + text.replace("\n\n", "\n\n\n", 3) + "\n/* trailing\n block */\n")
    assert bench.kernel_source_hash("qkv_decode.hip") == base
    # common.hpp is part of the stamp: a code change there voids it
    common = fake_root / "common.hpp"
    common.write_text(common.read_text() + "\nconstexpr int kUnusedProbe = 1;\n")
    assert bench.kernel_source_hash("qkv_decode.hip") != base
    common.write_text(common.read_text().replace("\nconstexpr int kUnusedProbe = 1;\n", ""))
    path.write_text(text.replace("namespace kaio {", "namespace kaio { constexpr int kProbe = 2;", 1))
    assert bench.kernel_source_hash("qkv_decode.hip") != base


def write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_from_counter_runs_and_calibration_copy(fake_root, tmp_path, capsys):
    kern = "void kaio::qkv_prefill_kernel<4, 8, 1, true, 128, 1>(kaio::QkvProblem, unsigned int)"
    other = "void kaio::qkv_prefill_kernel<4, 4, 1, true, 64, 2>(kaio::QkvProblem, unsigned int)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE: two instances per dispatch are summed; the copy reads half its bytes
    write_counters(tmp_path / "f", [(1, kern, "FETCH_SIZE", 600.0), (1, kern, "FETCH_SIZE", 400.0),
                                    (2, kern, "FETCH_SIZE", 1200.0), (3, other, "FETCH_SIZE", 9e9),
                                    (4, copy, "FETCH_SIZE", 131072.0), (5, copy, "FETCH_SIZE", 10.0)])
    write_counters(tmp_path / "w", [(1, kern, "WRITE_SIZE", 300.0), (2, kern, "WRITE_SIZE", 500.0),
                                    (4, copy, "WRITE_SIZE", 262144.0)])
    bench.write_traffic("qkv_prefill", "qkv_prefill.hip", str(tmp_path / "f"), str(tmp_path / "w"), "cmd")
    e = json.load(open(bench.TRAFFIC_FILE))["qkv_prefill"]
    assert e["fetch_kib_raw"] == 1100.0 and e["write_kib_raw"] == 400.0   # means over the kernel's dispatches
    assert e["fetch_scale"] == 2.0 and e["write_scale"] == 1.0             # the largest copy dispatch calibrates
    assert e["read_bytes_per_launch"] == 1100 * 2 * 1024 and e["write_bytes_per_launch"] == 400 * 1024
    assert e["bytes_per_launch"] == e["read_bytes_per_launch"] + e["write_bytes_per_launch"]
    assert e["dispatches"] == [2, 2] and e["source_hash"] == bench.kernel_source_hash("qkv_prefill.hip")
    # the bench uses the figure while the stamp matches, and drops it once the code changes
    assert bench.measured_traffic("qkv_prefill", "qkv_prefill.hip", 1.0) == e["bytes_per_launch"]
    p = fake_root / "qkv_prefill.hip"
    p.write_text(p.read_text().replace("namespace kaio {", "namespace kaio { constexpr int kProbe = 3;", 1))
    assert bench.measured_traffic("qkv_prefill", "qkv_prefill.hip", 1.0) is None
    assert bench.measured_traffic("qkv_decode", "qkv_decode.hip", 1.0) is None      # no entry
    # a run without the calibration copy is refused
    write_counters(tmp_path / "f2", [(1, kern, "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic("qkv_prefill", "qkv_prefill.hip", str(tmp_path / "f2"), str(tmp_path / "w"), "cmd")


def test_counter_summary_sums_instances_per_dispatch(tmp_path, capsys):
    kern = "void kaio::qkv_decode_kernel<4, 1, 1, 4, 16, true, 8>(kaio::QkvProblem, unsigned int)"
    write_counters(tmp_path / "c", [(1, kern, "SQ_INSTS_MFMA", 10.0), (1, kern, "SQ_INSTS_MFMA", 30.0),
                                    (2, kern, "SQ_INSTS_MFMA", 60.0), (1, kern, "GRBM_GUI_ACTIVE", 5.0),
                                    (2, kern, "GRBM_GUI_ACTIVE", 7.0)])
    bench.summarize([str(tmp_path / "c")])
    out = capsys.readouterr().out
    assert "(2 dispatches)" in out and "SQ_INSTS_MFMA=50" in out and "GRBM_GUI_ACTIVE=6" in out


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_trace_summary_groups_by_kernel_and_grid(tmp_path, capsys):
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Workgroup_Size_Y",
            "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
    rows = [("k<1>", 0, 5000, 256, 1, 1, 256 * 192, 1, 1), ("k<1>", 0, 7000, 256, 1, 1, 256 * 192, 1, 1),
            ("k<1>", 0, 6000, 256, 1, 1, 256 * 192, 1, 1), ("k<1>", 0, 9000, 256, 1, 1, 256 * 384, 1, 1)]
    os.makedirs(tmp_path / "t")
    with open(tmp_path / "t" / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)
    bench.summarize([str(tmp_path / "t")])
    out = capsys.readouterr().out
    # the three 192-workgroup dispatches: mean 6.00, min 5.00, median 6.00, max 7.00 us; the other grid apart
    assert "| k<1> | 192 x 256 | 3 | 6.00 | 5.00 | 6.00 | 7.00 |" in out
    assert "| k<1> | 384 x 256 | 1 | 9.00 | 9.00 | 9.00 | 9.00 |" in out

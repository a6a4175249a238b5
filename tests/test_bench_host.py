"""bench.py's host logic, on the CPU: the one-GPU refusal, the kernel-name keys of the
rocprofv3 summaries, the traffic summary's calibration on the copy probe, the derived SQ
counter ratios, and the rule that a traffic figure is reported only for the kernel source
it was measured on.  Synthetic rocprofv3 CSVs stand in for real runs."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FLAT = "void tq::(anonymous namespace)::tq_flat_kernel<8, 32, false>(tq::FlatArgs)"
FLAT4 = "void tq::(anonymous namespace)::tq_flat_kernel<8, 32, true>(tq::FlatArgs)"
PART = "void tq::(anonymous namespace)::tq_partition_kernel<8, 32, false>(tq::PartitionArgs)"
COPY = "probe_copy_kernel(unsigned char const*, unsigned char*, unsigned long)"


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


@pytest.mark.parametrize("name,key", [(FLAT, "tq_flat_kernel"), (FLAT4, "tq_flat_kernel[tq4]"),
                                      (PART, "tq_partition_kernel"), (COPY, "probe_copy_kernel"),
                                      ("tq_merge_kernel(tq::ReduceArgs)", "tq_merge_kernel")])
def test_kernel_keys(name, key):
    assert bench._kernel_key(name) == key


def test_traffic_summary_calibration(tmp_path):
    """FETCH_SIZE of the 1 GiB copy probe reads half its bytes (factor 2), WRITE_SIZE all of
    them (factor 1); a kernel's bytes per launch are its counters times those factors, and
    its average duration the trace's total over its calls."""
    prof = tmp_path / "prof"
    _write_csv(str(prof / "trace" / "trace_kernel_stats.csv"), [
        {"Name": FLAT, "Calls": 4, "TotalDurationNs": 4 * 336000.0, "MinNs": 330000.0, "MaxNs": 342000.0},
        {"Name": COPY, "Calls": 2, "TotalDurationNs": 2 * 460000.0, "MinNs": 450000.0, "MaxNs": 470000.0},
    ])
    _write_csv(str(prof / "fetch" / "fetch_counter_collection.csv"), [
        {"Kernel_Name": FLAT, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0},
        {"Kernel_Name": FLAT, "Counter_Name": "FETCH_SIZE", "Counter_Value": 1200.0},
        {"Kernel_Name": COPY, "Counter_Name": "FETCH_SIZE", "Counter_Value": 524288.0},
    ])
    _write_csv(str(prof / "write" / "write_counter_collection.csv"), [
        {"Kernel_Name": FLAT, "Counter_Name": "WRITE_SIZE", "Counter_Value": 2048.0},
        {"Kernel_Name": COPY, "Counter_Name": "WRITE_SIZE", "Counter_Value": 1048576.0},
    ])
    out = tmp_path / "out"
    bench.summarize_rocprof(str(prof), "wtest", out_dir=str(out))
    rec = json.loads((out / "traffic_tq_flat_kernel_wtest.json").read_text())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 1100 * 1024 * 2
    assert rec["write_bytes_per_launch"] == 2048 * 1024
    assert rec["hbm_bytes_per_launch"] == 1100 * 1024 * 2 + 2048 * 1024
    assert rec["avg_duration_us"] == 336.0
    assert rec["kernel_source_sha256"] == bench.kernel_sha()
    md = (out / "rocprof_wtest.md").read_text()
    assert "| tq_flat_kernel | 4 | 336.0 | 330.0 | 342.0 | 1100 | 2048 |" in md


def test_traffic_only_for_the_measured_source(tmp_path):
    rec = {"kernel": "tq_flat_kernel", "hbm_bytes_per_launch": 12345,
           "kernel_source_sha256": bench.kernel_sha()}
    p = tmp_path / "traffic_tq_flat_kernel_wtest.json"
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("wtest", "fused", profiles_dir=str(tmp_path)) == 12345
    rec["kernel_source_sha256"] = "0" * 64
    p.write_text(json.dumps(rec))
    assert bench.measured_traffic("wtest", "fused", profiles_dir=str(tmp_path)) is None
    assert bench.measured_traffic("other", "fused", profiles_dir=str(tmp_path)) is None


def test_counter_ratios(tmp_path):
    """Derived ratios from per-device counter sums: cycles = GRBM_GUI_ACTIVE / 8; waves per
    SIMD = 4 SQ_WAVE_CYCLES / 1024 / cycles; VALU busy = 4 SQ_ACTIVE_INST_VALU / 1024 /
    cycles; bank-conflict cycles = SQ_LDS_BANK_CONFLICT / 256 / cycles."""
    prof = tmp_path / "prof"
    cyc = 800000.0
    vals1 = {"SQ_WAVES": 2048, "SQ_WAVE_CYCLES": 2.0 * 1024 * cyc / 4, "SQ_BUSY_CYCLES": 1.0,
             "SQ_INSTS_VALU": 2048 * 100.0, "SQ_ACTIVE_INST_VALU": 0.5 * 1024 * cyc / 4,
             "SQ_INSTS_MFMA": 1.0, "SQ_VALU_MFMA_BUSY_CYCLES": 0.1 * 1024 * cyc,
             "SQ_INSTS_LDS": 1.0, "GRBM_GUI_ACTIVE": 8 * cyc}
    vals2 = {"SQ_LDS_BANK_CONFLICT": 0.03 * 256 * cyc, "SQ_ACTIVE_INST_LDS": 1.0,
             "SQ_WAIT_INST_ANY": 1.0, "SQ_WAIT_ANY": 1.0, "SQ_INSTS_SALU": 1.0,
             "SQ_ACTIVE_INST_ANY": 1.0, "GRBM_GUI_ACTIVE": 8 * cyc}
    for sub, vals in (("pmc1", vals1), ("pmc2", vals2)):
        _write_csv(str(prof / sub / f"{sub}_counter_collection.csv"),
                   [{"Kernel_Name": FLAT, "Counter_Name": c, "Counter_Value": v} for c, v in vals.items()])
    out = tmp_path / "out"
    bench.summarize_counters(str(prof), "wtest", out_dir=str(out))
    md = (out / "counters_wtest.md").read_text()
    assert "| tq_flat_kernel | 8e+05 | 2.00 | 50.0 % | 10.0 % | 3.0 % | 100 |" in md

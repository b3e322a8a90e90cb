"""Host logic of bench.py on the CPU: the rocprofv3 summaries and the HBM
traffic scale computed from hand-made counter files, and the lookup that
the roofline's `traffic` field reads them back with."""
import csv
import json
import os

import pytest

import bench

GATEUP = "void moe::(anonymous namespace)::expert_gemm<0, 64, 256, 64, 2, 4, 4, 0, 0, 64, 4>(moe::ExpertArgs)"
DOWN = "void moe::(anonymous namespace)::expert_gemm<1, 64, 256, 64, 2, 4, 3, 0, 0, 64, 3>(moe::ExpertArgs)"
COPY = "__amd_rocclr_copyBuffer"
GIB = 1073741824


def _counter_csv(path, rows):
    """rows: (kernel name, counter, value) per dispatch."""
    os.makedirs(path)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (k, c, v) in enumerate(rows):
            w.writerow([i + 1, k, c, v])


@pytest.fixture
def prof(tmp_path):
    d = tmp_path / "prof"
    # kernel trace: rocprofv3's per-kernel statistics
    os.makedirs(d / "kt_decode")
    with open(d / "kt_decode" / "run_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow([GATEUP, 10, 1500000, 150000.0, 60.0, 140000, 160000, 1.0])
        w.writerow([DOWN, 10, 800000, 80000.0, 32.0, 75000, 85000, 1.0])
    # a 1 GiB copy that the counters report as 1.25x its bytes read and
    # 0.5x its bytes written (in KiB)
    _counter_csv(str(d / "pmc_fetch_copy"), [(COPY, "FETCH_SIZE", 1.25 * GIB / 1024)] * 5)
    _counter_csv(str(d / "pmc_write_copy"), [(COPY, "WRITE_SIZE", 0.5 * GIB / 1024)] * 5)
    # two launches of each kernel: the mean per launch is what counts
    _counter_csv(str(d / "pmc_fetch_decode"), [(GATEUP, "FETCH_SIZE", 1000.0),
                                               (GATEUP, "FETCH_SIZE", 3000.0),
                                               (DOWN, "FETCH_SIZE", 500.0),
                                               (COPY, "FETCH_SIZE", 9e9)])
    _counter_csv(str(d / "pmc_write_decode"), [(GATEUP, "WRITE_SIZE", 10.0),
                                               (GATEUP, "WRITE_SIZE", 30.0),
                                               (DOWN, "WRITE_SIZE", 40.0)])
    return str(d), str(tmp_path / "out")


def test_traffic_scaled_by_the_copy_calibration(prof):
    d, out = prof
    bench.summarize_profiles(d, out)
    t = json.load(open(os.path.join(out, "traffic.json")))
    gu, dn = t["gateup_kernel:decode"], t["down_kernel:decode"]
    # mean FETCH 2000 KiB, scaled by 1/1.25; mean WRITE 20 KiB, scaled by 1/0.5
    assert gu["read_bytes"] == pytest.approx(2000 * 1024 / 1.25)
    assert gu["write_bytes"] == pytest.approx(20 * 1024 / 0.5)
    assert gu["bytes_per_launch"] == pytest.approx(2000 * 1024 / 1.25 + 20 * 1024 / 0.5)
    assert dn["read_bytes"] == pytest.approx(500 * 1024 / 1.25)
    assert gu["kernel"] == "expert_gemm<0, 64, 256, 64, 2, 4, 4, 0, 0, 64, 4>"
    # non-library kernels are left out
    assert not any(COPY in k for k in t if k != "calibration")
    md = open(os.path.join(out, "hbm_traffic.md")).read()
    assert f"{2000 * 1024 / 1.25 / 1e6:.1f}" in md


def test_kernel_trace_summary(prof):
    d, out = prof
    bench.summarize_profiles(d, out)
    md = open(os.path.join(out, "kernels_decode.md")).read()
    assert "| `expert_gemm<0, 64, 256, 64, 2, 4, 4, 0, 0, 64, 4>` | 10 | 150.00 | 140.00 | 160.00 | 60.0% |" in md
    assert bench.PROFILE_COMMANDS["kt_decode"] in md


def test_traffic_lookup_follows_the_kernel_source(prof):
    d, out = prof
    bench.summarize_profiles(d, out)
    assert bench.traffic_for("gateup_kernel", "decode", out) == pytest.approx(
        2000 * 1024 / 1.25 + 20 * 1024 / 0.5)
    assert bench.traffic_for("gateup_kernel", "prefill", out) is None
    # counters taken on another version of the kernel source are not used
    path = os.path.join(out, "traffic.json")
    t = json.load(open(path))
    t["gateup_kernel:decode"]["source_sha256"] = "0" * 64
    json.dump(t, open(path, "w"))
    assert bench.traffic_for("gateup_kernel", "decode", out) is None


def test_source_hash_sees_code_not_comments():
    src = "// header\nint f(int a) {  // the sum\n  /* two\n lines */ return a + 1;\n}\n"
    assert bench._code_only(src) == bench._code_only(
        "// another header\n\nint f(int a) {\n  return a + 1;  /* one */\n}\n")
    assert bench._code_only(src) != bench._code_only(src.replace("a + 1", "a + 2"))
    assert bench._code_only("int c = 6 / 2;  // half") == "int c = 6 / 2;"

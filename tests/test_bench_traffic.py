"""Host logic of the bench's HBM-traffic record (no GPU): the counters of each kernel are
scaled by what the same counter reads for a 1 GiB calibration copy, then averaged over
launches."""
import csv
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Counter_Name", "Kernel_Name", "Counter_Value"]


def _csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for name, value in rows:
            w.writerow({"Counter_Name": counter, "Kernel_Name": name, "Counter_Value": value})


def test_traffic_record_scales_by_the_calibration_copy(tmp_path):
    part = "void cqsa::(anonymous namespace)::attn_partial_bf16<128>(cqsa::(anonymous namespace)::AttnParams)"
    merge = "void cqsa::(anonymous namespace)::merge_partials<128, unsigned short>(cqsa::(anonymous namespace)::MergeParams)"
    copy = "__amd_rocclr_copyBuffer"
    # FETCH_SIZE reads half of the bytes (factor 2), WRITE_SIZE all of them
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [(copy, 524288.0), (copy, 12.0), (part, 1000.0), (part, 1002.0),
                                             (merge, 300.0), (merge, 300.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [(copy, 1048576.0), (part, 700.0), (part, 700.0),
                                             (merge, 100.0), (merge, 102.0)])
    rec = bench.traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "0123456789abcdef")
    assert rec["calibration"]["fetch_scale"] == 2.0 and rec["calibration"]["write_scale"] == 1.0
    assert rec["hbm_bytes_read_per_launch"] == 1001 * 1024 * 2
    assert rec["hbm_bytes_written_per_launch"] == 700 * 1024
    assert rec["hbm_bytes_per_launch"] == (1001 * 2 + 700) * 1024
    assert rec["merge"]["hbm_bytes_per_launch"] == (300 * 2 + 101) * 1024
    assert rec["kernel_source_sha256_16"] == "0123456789abcdef"


def test_traffic_record_needs_the_calibration_copy(tmp_path):
    _csv(tmp_path / "f.csv", "FETCH_SIZE", [("attn_partial_bf16<128>", 1.0), ("merge_partials<128", 1.0)])
    _csv(tmp_path / "w.csv", "WRITE_SIZE", [("attn_partial_bf16<128>", 1.0), ("merge_partials<128", 1.0)])
    with pytest.raises(ValueError):
        bench.traffic_record(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "x")



def test_copy_summary_takes_the_union_of_copy_intervals(tmp_path):
    # two host-to-device copies overlapping on two streams count once; device-to-host apart
    path = tmp_path / "copies.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kind", "Direction", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, b, e in [("MEMORY_COPY_HOST_TO_DEVICE", 0, 4_000_000), ("MEMORY_COPY_HOST_TO_DEVICE", 1_000_000, 6_000_000),
                        ("MEMORY_COPY_HOST_TO_DEVICE", 10_000_000, 11_000_000),
                        ("MEMORY_COPY_DEVICE_TO_HOST", 2_000_000, 3_000_000),
                        ("MEMORY_COPY_DEVICE_TO_HOST", 5_000_000, 7_000_000),
                        ("MEMORY_COPY_DEVICE_TO_DEVICE", 0, 9_000_000)]:
            w.writerow({"Kind": "MEMORY_COPY", "Direction": d, "Start_Timestamp": b, "End_Timestamp": e})
    out = bench.copy_summary(str(path))
    assert out["h2d"] == {"copies": 3, "busy_ms": 7.0, "span_ms": 11.0}
    assert out["d2h"] == {"copies": 2, "busy_ms": 3.0, "span_ms": 5.0}


def test_copy_summary_counts_only_the_given_streams(tmp_path):
    # copies on stream 0 (the bench's own) are left out when the engine's streams are named
    path = tmp_path / "copies.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kind", "Direction", "Stream_Id", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for d, sid, b, e in [("MEMORY_COPY_HOST_TO_DEVICE", "0", 0, 5_000_000),
                             ("MEMORY_COPY_HOST_TO_DEVICE", "1", 1_000_000, 3_000_000),
                             ("MEMORY_COPY_HOST_TO_DEVICE", "2", 2_000_000, 4_000_000),
                             ("MEMORY_COPY_DEVICE_TO_HOST", "2", 6_000_000, 7_000_000),
                             ("MEMORY_COPY_DEVICE_TO_HOST", "0", 8_000_000, 12_000_000)]:
            w.writerow({"Kind": "MEMORY_COPY", "Direction": d, "Stream_Id": sid, "Start_Timestamp": b,
                        "End_Timestamp": e})
    out = bench.copy_summary(str(path), {"1", "2"})
    assert out["h2d"] == {"copies": 2, "busy_ms": 3.0, "span_ms": 3.0}
    assert out["d2h"] == {"copies": 1, "busy_ms": 1.0, "span_ms": 1.0}
    every = bench.copy_summary(str(path))
    assert every["h2d"]["busy_ms"] == 5.0 and every["d2h"]["busy_ms"] == 5.0


def test_bench_refuses_more_than_one_gpu():
    """The bench runs on one GPU: --gpus 2 exits with status 2 and says why, before any
    GPU or torch use."""
    import subprocess
    proc = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                          capture_output=True, text=True, timeout=120)
    assert proc.returncode == 2
    assert "one GPU" in proc.stderr and proc.stdout == ""

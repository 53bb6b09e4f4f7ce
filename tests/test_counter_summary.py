"""The profile summariser (joint_video_audio_amd.counter_summary) on small
hand-written CSVs: averages per dispatch, role split by launch order, exact
name matching and the copy-kernel scale."""
import csv
import os
import subprocess
import sys

from joint_video_audio_amd import counter_summary as cs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_roles_and_exact_names(tmp_path):
    p = tmp_path / "c.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = []
    # k_gemm_bf16<1> launched as output (dispatches 1, 5) and down (3, 7); a
    # counter split over two rows of one dispatch adds up
    for d, v in ((1, 10.0), (3, 30.0), (5, 14.0), (7, 34.0)):
        rows += [[d, "void k_gemm_bf16<1>(int)", "X", v / 2], [d, "void k_gemm_bf16<1>(int)", "X", v / 2]]
    rows += [[2, "void k_gemm_bf16_half<1>(int)", "X", 99.0], [4, "copyBuffer", "X", 2048.0]]
    write(p, hdr, rows)
    out, _ = cs.per_dispatch(str(p), "k_gemm_bf16<1>", 2, 0)
    assert out == {"X": 12.0}
    out, _ = cs.per_dispatch(str(p), "k_gemm_bf16<1>", 2, 1)
    assert out == {"X": 32.0}
    out, _ = cs.per_dispatch(str(p), "k_gemm_bf16")  # substring: both kernels
    assert out == {"X": (10 + 30 + 14 + 34 + 99) / 5}
    out, _ = cs.per_dispatch(str(p), "=void k_gemm_bf16_half<1>(int)")
    assert out == {"X": 99.0}
    r = subprocess.run([sys.executable, "-m", "joint_video_audio_amd.counter_summary", str(p), "k_gemm_bf16_half",
                        "4194304"], capture_output=True, text=True, cwd=ROOT, check=True)
    # 4 MiB copy read as 2048 KiB: 4194304 / (2048 * 1024) = 2.0
    assert "bytes/(KiB*1024) = 2.0000" in r.stdout


def test_trace_durations(tmp_path):
    p = tmp_path / "t.csv"
    hdr = ["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    write(p, hdr, [[1, "k_gemm_bf16", 0, 100], [2, "k_gemm_bf16_half", 100, 130], [3, "k_gemm_bf16", 200, 500],
                   [4, "k_gemm_bf16", 600, 700], [5, "k_gemm_bf16", 800, 1300]])
    assert cs.mean_duration_ns(str(p), "=k_gemm_bf16", 2, 0) == (100.0, 2)
    assert cs.mean_duration_ns(str(p), "=k_gemm_bf16", 2, 1) == (400.0, 2)
    assert cs.mean_duration_ns(str(p), "k_gemm_bf16") == ((100 + 30 + 300 + 100 + 500) / 5, 5)
    r = subprocess.run([sys.executable, "-m", "joint_video_audio_amd.counter_summary", str(p), "=k_gemm_bf16_half"],
                       capture_output=True, text=True, cwd=ROOT, check=True)
    assert "1 dispatches, average duration 30 ns" in r.stdout

"""Host logic of bench.py, on the CPU: the one-GPU refusal, and the readers
and writers of the rocprofv3 summaries under profiles/ (counter calibration
on the copy of known size, the per-launch HBM bytes the bench line quotes,
and the rule that a summary taken before a kernel's source changed is not
used).  Synthetic counter tables stand in for rocprofv3's CSV output; nothing
here needs a GPU or the HIP library."""
import csv
import os
import re
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECODE = "pa::decode_kernel<pa::BF16, 1, 128, true, false>(pa::(anonymous namespace)::DecodeArgs)"
COPY = "void at::native::elementwise_kernel_manual_unroll<128, 4, direct_copy_kernel_cuda>(int, F)"


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_traffic_is_read_only_from_a_summary_of_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    cur = bench.source_hash(bench.KERNEL_SOURCES["decode_kernel"])
    assert bench.traffic_from_profiles("decode_kernel", "w") is None  # no summary
    (tmp_path / "decode_kernel.w.pmc.md").write_text(f"hbm_bytes_per_launch: 1.5e+09\nsource_sha256_16: {cur}\n")
    assert bench.traffic_from_profiles("decode_kernel", "w") == 1.5e9
    stale = "0" * 16 if cur != "0" * 16 else "1" * 16
    (tmp_path / "decode_kernel.w.pmc.md").write_text(f"hbm_bytes_per_launch: 1.5e+09\nsource_sha256_16: {stale}\n")
    assert bench.traffic_from_profiles("decode_kernel", "w") is None


def test_counter_summary_calibrates_on_the_copy_and_round_trips(tmp_path, monkeypatch):
    """Two decode dispatches read 1000 and 3000 KiB by FETCH_SIZE and wrote
    10 and 30 KiB by WRITE_SIZE; the leg's copy of CAL_BYTES shows up at half
    its size in FETCH_SIZE and at its size in WRITE_SIZE.  So the kernel read
    2000 KiB / 0.5 and wrote 20 KiB / 1.0 per launch on average."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    os.makedirs(bench.PROFILES)
    cal_kib = bench.CAL_BYTES / 1024
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # FETCH_SIZE is the sum of several counter instances: two rows per dispatch
    _write_csv(str(tmp_path / "f" / "run_counter_collection.csv"), hdr,
               [[1, DECODE, "FETCH_SIZE", 400], [1, DECODE, "FETCH_SIZE", 600], [2, DECODE, "FETCH_SIZE", 3000],
                [3, COPY, "FETCH_SIZE", cal_kib * 0.5], [4, COPY, "FETCH_SIZE", 7.0]])
    _write_csv(str(tmp_path / "w" / "run_counter_collection.csv"), hdr,
               [[1, DECODE, "WRITE_SIZE", 10], [2, DECODE, "WRITE_SIZE", 30], [3, COPY, "WRITE_SIZE", cal_kib]])
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), "decode_kernel", "w",
                        "rocprofv3 --pmc COUNTER -- python3 bench.py")
    text = open(os.path.join(bench.PROFILES, "decode_kernel.w.pmc.md")).read()
    want = 2000 * 1024 / 0.5 + 20 * 1024 / 1.0
    got = float(re.search(r"hbm_bytes_per_launch:\s*([0-9.e+]+)", text).group(1))
    assert got == pytest.approx(want, rel=1e-6)
    assert "--pmc FETCH_SIZE" in text and "--pmc WRITE_SIZE" in text
    assert bench.traffic_from_profiles("decode_kernel", "w") == pytest.approx(want, rel=1e-6)


def test_kernel_time_summary_table(tmp_path):
    _write_csv(str(tmp_path / "t" / "run_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[f"void {DECODE}", 4, 541000.0, 530000.0, 560000.0, 61.25]])
    out = str(tmp_path / "step.w.kernel_stats.md")
    bench.summarize_trace(str(tmp_path / "t"), out, "rocprofv3 --kernel-trace --stats -- python3 bench.py")
    text = open(out).read()
    assert "| `pa::decode_kernel<pa::BF16, 1, 128, true, false>` | 4 | 541.00 | 530.00 | 560.00 | 61.2% |" in text
    assert "`rocprofv3 --kernel-trace --stats -- python3 bench.py`" in text

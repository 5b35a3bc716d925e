"""Measurement tooling on the CPU: bench.py's one-GPU contract and the
rocprofv3 summarizer that writes profiles/ (kernel-name filtering, the last-N
selection, the copy calibration of the HBM counters)."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

GEMV = "void wq::(anonymous namespace)::gemv_kernel<0, 4, 1, 1, 1, 4, 2, false, 1, false>(wq::(anonymous namespace)::GemvArgs)"
OTHER = "void wq::(anonymous namespace)::gemv_kernel<0, 4, 1, 2, 1, 0, 2, false, 1, true>(wq::(anonymous namespace)::GemvArgs)"
COPY = "__amd_rocclr_copyBuffer"


def run(*args):
    return subprocess.run([sys.executable, *args], capture_output=True, text=True, cwd=ROOT, timeout=300)


def test_bench_measures_one_gpu():
    r = run("bench.py", "--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def write_trace(path, rows):
    cols = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X",
            "Grid_Size_Y"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(cols)
        for name, start, dur_ns, grid in rows:
            w.writerow(["KERNEL_DISPATCH", name, start, start + dur_ns, 256, grid, 1])


def test_trace_summary_filters_by_kernel_name_and_keeps_the_last(tmp_path):
    d = tmp_path / "t"
    d.mkdir()
    # same grid, different kernels: they must not be merged; the first two
    # GEMV dispatches (warm-up) are dropped by --last 3
    rows = [(GEMV, 1000 * i, ns, 4096) for i, ns in enumerate([50000, 40000, 10000, 12000, 11000])]
    rows += [(OTHER, 10 ** 7 + i, 99000, 4096) for i in range(3)]
    write_trace(d / "trace_kernel_trace.csv", rows)
    r = run("prof_summary.py", "trace", "--run", "case", str(d), "--last", "3", "--alg", "case", "22000000")
    assert r.returncode == 0, r.stderr
    gemv = [l for l in r.stdout.splitlines() if "gemv_kernel<0, 4, 1, 1, 1" in l]
    other = [l for l in r.stdout.splitlines() if "gemv_kernel<0, 4, 1, 2, 1" in l]
    assert len(gemv) == 1 and len(other) == 1
    cells = [c.strip() for c in gemv[0].split("|")]
    assert cells[5] == "3"                  # dispatches kept
    assert cells[6] == "11.000"             # average of 10, 12, 11 us
    assert cells[7] == "11.000"             # median
    assert cells[8].startswith("2000.0 GB/s")  # 22 MB / 11 us
    assert "Summary command" in r.stdout and "--last 3" in r.stdout


def write_pmc(path, counter, rows):
    cols = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
            "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(cols)
        for i, (name, grid, value) in enumerate(rows):
            w.writerow([i, grid, name, counter, value, 1000 * i, 1000 * i + 500])


def test_counter_summary_calibrates_with_the_largest_copy(tmp_path):
    fetch, write = tmp_path / "p1", tmp_path / "p2"
    fetch.mkdir()
    write.mkdir()
    mib256 = 1 << 18  # KiB in 256 MiB
    # the copy kernel also serves small uploads (small grid): only the
    # largest-grid dispatches calibrate; FETCH_SIZE reads half the bytes
    write_pmc(fetch / "pmc_counter_collection.csv", "FETCH_SIZE",
              [(COPY, 1024, 7.0), (GEMV, 4096, 5000.0), (GEMV, 4096, 5000.0), (COPY, 1 << 20, mib256 / 2)])
    write_pmc(write / "pmc_counter_collection.csv", "WRITE_SIZE",
              [(COPY, 1024, 3.0), (GEMV, 4096, 20.0), (GEMV, 4096, 20.0), (COPY, 1 << 20, mib256)])
    r = run("prof_summary.py", "pmc", "--run", "case", str(fetch), "--run", "case", str(write),
            "--alg", "case", "10000000", "--traffic-of", "case", "--traffic-kernel", "gemv_kernel<0, 4, 1, 1")
    assert r.returncode == 0, r.stderr
    assert "factor 0.5000" in r.stdout and "factor 1.0000" in r.stdout
    # (5000 / 0.5 + 20) KiB
    want = (5000 * 1024) * 2 + 20 * 1024
    assert f"- hbm_bytes_per_launch: {want}" in r.stdout
    assert f"{want / 10000000:.4f} x the algorithmic" in r.stdout

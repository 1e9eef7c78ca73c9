"""Host-side checks of bench.py's profile summarizers (no GPU): the kernel-statistics
summary with trace medians, and the HBM-traffic scaling by a copy of known size."""

import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_ALL)
        w.writerow(header)
        w.writerows(rows)


def _bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    return r.stdout


def test_stats_summary_reports_trace_medians(tmp_path):
    stats = tmp_path / "k_stats.csv"
    trace = tmp_path / "k_trace.csv"
    _write_csv(stats, ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
               [["kern_a", 3, 2000.0, 1000.0, 4000.0], ["kern_b", 1, 5000.0, 5000.0, 5000.0]])
    # kern_a: durations 1, 1.5 and 4 us (median 1.5, mean 2.17); kern_b: 5 us
    _write_csv(trace, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [["kern_a", 0, 1000], ["kern_a", 10000, 11500], ["kern_a", 20000, 24000], ["kern_b", 0, 5000]])
    out = _bench("--summarize-stats", str(stats), "the command", str(trace))
    lines = [l for l in out.splitlines() if l.strip().startswith("kern_")]
    assert "# command: the command" in out and "median_us" in out
    a = lines[0].split()
    assert a[0] == "kern_a" and a[1] == "3" and float(a[2]) == 2.0 and float(a[-1]) == 1.5
    assert lines[1].split()[-1] == "5.000"
    # without a trace there is no median column
    assert "median_us" not in _bench("--summarize-stats", str(stats), "cmd")


def test_traffic_summary_scales_by_the_copy(tmp_path):
    """FETCH_SIZE of the copy reads half its bytes (factor 2), WRITE_SIZE all (factor 1):
    a kernel reading 1000 KiB raw and writing 10 KiB moves (2000 + 10) KiB."""
    copy_kib = (256 << 20) // 1024
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    _write_csv(fetch, hdr, [["copyBuffer", "FETCH_SIZE", copy_kib / 2], ["kern<1>", "FETCH_SIZE", 1000.0],
                            ["kern<1>", "FETCH_SIZE", 1000.0]])
    _write_csv(write, hdr, [["copyBuffer", "WRITE_SIZE", copy_kib], ["kern<1>", "WRITE_SIZE", 10.0]])
    out = _bench("--summarize-pmc", str(fetch), str(write), "gemv_mt_kernel", "cf", "cw")
    # the kernel name filter: no row matches "gemv_mt_kernel", so nothing is scaled
    assert "hbm_bytes_per_launch" not in out
    _write_csv(fetch, hdr, [["copyBuffer", "FETCH_SIZE", copy_kib / 2], ["gemv_mt_kernel<2, 1>", "FETCH_SIZE", 1000.0]])
    _write_csv(write, hdr, [["copyBuffer", "WRITE_SIZE", copy_kib], ["gemv_mt_kernel<2, 1>", "WRITE_SIZE", 10.0]])
    out = _bench("--summarize-pmc", str(fetch), str(write), "gemv_mt_kernel", "cf", "cw")
    kv = dict(l.split(": ", 1) for l in out.splitlines() if ": " in l and not l.startswith("#"))
    assert float(kv["fetch_scale"]) == 2.0 and float(kv["write_scale"]) == 1.0
    assert int(kv["hbm_bytes_per_launch"]) == (2000 + 10) * 1024

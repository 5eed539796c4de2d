"""Host logic of the bench harness, on the CPU: its byte accounting against figures worked out
by hand from the workload shapes, the filtering and scaling of the profile summaries it writes,
the source hash that marks a summary stale, and its refusal of more than one GPU."""
import csv
import os
import re
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


# Bytes a step must move: x, delta and y at B*L*D elements, B and C at B*L*N, A and h_final at
# D*N fp32 (decode: the state read and written, the token rows, and A, per layer).  The figures
# are the workload table's, computed by hand from the shapes:
#   4K:   3*4096*8192*2 + 2*4096*16*2 + 2*8192*16*4
#   64K:  3*65536*8192*2 + 2*65536*16*2 + 2*8192*16*4
#   256K: 3*262144*8192*2 + 2*262144*16*2 + 2*8192*16*4
#   decode, 28 layers of: 2*256*8192*16*4 + 3*256*8192*2 + 2*256*16*2 + 8192*16*4
@pytest.mark.parametrize("name,expected", [
    ("prefill_4k", 202_637_312),
    ("prefill_64k", 3_226_468_352),
    ("prefill_256k", 12_902_727_680),
    ("decode_256x28", 28 * 281_559_040),
])
def test_algorithmic_bytes_match_the_hand_counts(name, expected):
    assert bench.algorithmic_bytes(workloads.get(name)) == expected


def test_trapezoid_and_mimo_bytes_add_their_extra_inputs():
    wl = workloads.get("prefill_64k")
    base = bench.algorithmic_bytes(wl)
    tokens = wl.batch * wl.L
    # the trapezoidal rule also reads lam, one more [L][D] bf16 tensor
    assert bench.algorithmic_bytes(wl, trapezoid=True) - base == tokens * wl.D * 2
    # rank R: x and y hold R values per channel, B and C N x R
    R = 4
    extra = 2 * (R - 1) * tokens * wl.D * 2 + 2 * (R - 1) * tokens * wl.N * 2
    assert bench.algorithmic_bytes(wl, mimo=R) - base == extra


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_trace_summary_skips_warmup_and_short_launches(tmp_path):
    name = "void jscan::prefill_rows_kernel<x>(int)"
    durations_us = [500, 400, 300]          # warm-up launches
    durations_us += [2, 100, 110, 120, 130, 140]   # one short check launch among the timed ones
    rows, t = [], 1_000_000
    for d in durations_us:
        rows.append([name, t, t + d * 1000])
        t += d * 1000 + 5_000
    rows.append(["other_kernel", t, t + 7_000])
    _write_csv(tmp_path / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    out = bench.trace_summary(str(tmp_path), warmup=3)
    line = out[out.index(name):].splitlines()[1]
    assert "launches 9" in line and "(and 1 short ones)" in line
    assert "median 120.0 us" in line and "min 100.0" in line and "max 140.0" in line


def test_counter_summary_scales_by_the_copy_calibration_and_drops_short_dispatches(tmp_path):
    name = "void jscan::prefill_rows_kernel<jscan::BF16, false>(int)"
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    fetch_kib, write_kib = [1.0e6, 1.2e6], [1.1e6, 1.1e6]
    for sub, counter, vals in (("f", "FETCH_SIZE", fetch_kib), ("w", "WRITE_SIZE", write_kib)):
        d = tmp_path / sub
        d.mkdir()
        rows = [[1, name, counter, 5.0, 0, 10_000]]   # the short check dispatch
        for i, v in enumerate(vals):
            # a counter may come in several rows per dispatch (one per instance): they add up
            rows.append([2 + i, name, counter, v / 2, 100_000, 2_100_000])
            rows.append([2 + i, name, counter, v / 2, 100_000, 2_100_000])
        _write_csv(d / "run_counter_collection.csv", header, rows)
    args = types.SimpleNamespace(workload="prefill_64k", mimo=0, trapezoid=False, scalar_a=False)
    out = bench.counter_summary(args, str(tmp_path / "f"), str(tmp_path / "w"))
    vals = dict(re.findall(r"^(\w+) = (\S+)", out, flags=re.M))
    cal = dict(re.findall(r"^\s*(\w+)\s*=\s*([0-9.eE+-]+)\s*$",
                          open(os.path.join(ROOT, "profiles", "counters_copy_calibration.txt")).read(), flags=re.M))
    fetch_scale = (1 << 20) / float(cal["copy_fetch_KiB_per_GiB"])
    write_scale = (1 << 20) / float(cal["copy_write_KiB_per_GiB"])
    assert vals["dispatches_fetch"] == "2" and vals["dispatches_write"] == "2"
    rd = sum(fetch_kib) / 2 * 1024 * fetch_scale
    wr = sum(write_kib) / 2 * 1024 * write_scale
    assert float(vals["hbm_read_bytes_per_launch"]) == pytest.approx(rd, rel=1e-5)
    assert float(vals["hbm_write_bytes_per_launch"]) == pytest.approx(wr, rel=1e-5)
    assert int(vals["algorithmic_bytes_per_launch"]) == 3_226_468_352
    assert float(vals["traffic_over_algorithmic"]) == pytest.approx((rd + wr) / 3_226_468_352, abs=1e-4)


def test_source_hash_ignores_comments_and_spacing():
    a = "int f(int x) {  // the sum\n    return x + 1;   /* one more */\n}\n"
    b = "int f(int x) {\n  return x + 1;\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(b.replace("+ 1", "+ 2"))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

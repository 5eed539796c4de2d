#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_64k]

One step is one full pass of the hot path over one batch: a jscan_prefill of the whole
sequence (prefill workloads) or one decode token through all layers (decode workload).
Inputs are generated once, moved to HBM, and stay resident; the timed region holds only
the library's kernels, bracketed by stream synchronisation and timed with HIP events on
the stream the kernels run on.  Prints exactly one JSON line.

The line's `roofline` is the metric's: HBM, algorithmic bytes of a launch of the dominant
kernel over its average launch time (HIP events), against 8 TB/s.  `roofline_alu` puts the
same launch against the vector-ALU bound that actually binds the prefill.  That bound comes
from the committed microbenchmarks (profiles/micro_gfx950.txt, `bench.py --micro`): a SIMD
retires a 64-lane fp32 FMA-class instruction every FMA_CYCLES and an exponential every
EXP_CYCLES (about 3 FMA slots) when enough waves feed it.  A state element of the S6 scan
needs an exponent product, the exponential, the input product and two fused multiply-adds,
4 + EXP_SLOTS slots, 7 flops; at the 2.4 GHz peak engine clock over 256 CUs x 4 SIMDs that is
about 8.6e12 state elements/s (1.0 ms for the 64K x 8192 scan, 40% of the HBM peak).  The
other forms count their own instructions the same way: a scaled-identity A evaluates the decay
once per 16 states; a complex state adds the rotation (a sine and a cosine, each costed like
the exponential); the exponential-trapezoidal rule adds one FMA per element and reads lam; a
rank-R MIMO scan makes the input term a rank-R sum and the output R FMAs per element.  None of
these counts includes the instructions that deliver operands between lanes (DPP broadcasts,
permlane swaps), which the kernels also need.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "selective-scan elems/s (B·L·D) + HBM GB/s % of peak, L=64K D=8192 N=16"
HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0                # dense bf16 matrix-core peak of MI355X
PRODUCER_RANK = 256                           # rank of delta's projection (d_model 4096 / 16)


def _micro_rates():
    """Cycles per wave instruction of a SIMD running 8 waves, for the fused multiply-add and the
    base-2 exponential, from the committed microbenchmark summary (bench.py --micro); the
    values measured on the MI355X when it is absent."""
    fma, exp = 2.59, 7.91
    path = os.path.join(ROOT, "profiles", "micro_gfx950.txt")
    if os.path.exists(path):
        for line in open(path):
            if line.startswith("valu_cycles_per_wave_instruction.fma.cycles_per_instr_8w ="):
                fma = float(line.split("=")[1])
            elif line.startswith("valu_cycles_per_wave_instruction.exp.cycles_per_instr_8w ="):
                exp = float(line.split("=")[1])
    return fma, exp


# The vector-ALU bound of the scans.  A SIMD retires one wave-wide (64-lane) FMA-class instruction
# per FMA_CYCLES and one exponential (or sine, cosine) per EXP_CYCLES when enough waves feed it,
# measured by the microbenchmarks; at MI355X's 2.4 GHz peak engine clock that is
# VALU_SLOTS_PER_S FMA-class lane-instructions per second over 256 CUs x 4 SIMDs, and a
# transcendental costs EXP_SLOTS of them.  The counts below are the instructions the
# arithmetic needs per state element, with no operand-delivery (DPP, permlane) overhead.
FMA_CYCLES, EXP_CYCLES = _micro_rates()
VALU_SLOTS_PER_S = 256 * 4 * 64 * 2.4e9 / FMA_CYCLES
EXP_SLOTS = EXP_CYCLES / FMA_CYCLES
SLOTS_PER_STATE_ELEM = 4 + EXP_SLOTS          # mul, exp, mul, fma, fma
FLOPS_PER_STATE_ELEM = 7                      # mul 1 + exp 1 + mul 1 + fma 2 + fma 2
PEAK_STATE_ELEMS = VALU_SLOTS_PER_S / SLOTS_PER_STATE_ELEM
SCALAR_A_SLOTS = 3 + (1 + EXP_SLOTS) / 16     # mul, fma, fma; decay (mul + exp) once per 16 states
SCALAR_A_FLOPS = 5 + 2 / 16
# complex state, per real component (half a complex state): decay mul + exp, angle mul + fract,
# cos and sin, r cos and r sin, two input products, four fma, y (2)
COMPLEX_A_SLOTS = (1 + EXP_SLOTS + 2 + 2 * EXP_SLOTS + 2 + 2 + 4 + 2) / 2
COMPLEX_A_FLOPS = 21 / 2
TRAP_SLOTS, TRAP_FLOPS = 1, 2                 # the left end point's fma, on top of the form's count


def mimo_cost(form: str, R: int):
    """(issue slots, flops) per state element of the rank-R scan; R = 1 gives the single-input counts."""
    if form == "scalar":
        return 2 * R + 1 + (1 + EXP_SLOTS) / 16, 4 * R + 1 + 2 / 16
    if form == "complex":
        return (11 + 3 * EXP_SLOTS + 4 * R) / 2, (8 * R + 13) / 2
    return 2 * R + 3 + EXP_SLOTS, 4 * R + 3


KERNEL_SOURCES = {
    "prefill": ["scan_update.h", "mfma_common.h", "prefill_rows_kernel.h"],
    "step": ["scan_update.h", "step_kernel.h"],
    "prefill_mimo": ["scan_update.h", "mfma_common.h", "prefill_rows_kernel.h", "step_kernel.h", "mimo_kernels.h",
                     "prefill_mimo_rows_kernel.h"],
    "step_mimo": ["scan_update.h", "step_kernel.h", "mimo_kernels.h"],
    "producer": ["scan_update.h", "mfma_common.h", "project_kernels.h"],
}


def _code_only(text: str) -> str:
    """C++ source with comments and blank space removed: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(kind: str) -> str:
    """Hash of the code of one kernel's sources (a key of KERNEL_SOURCES, comments left out); a
    profile summary records it, and its counters count only while that code is unchanged."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "mamba_selective_scan_03_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, trapezoid: bool = False, mimo: int = 0) -> int:
    """Bytes a step must move at least.  The trapezoidal rule also reads lam (like delta) and,
    in decode, the previous token's x and B rows.  A rank-R MIMO scan has R values per channel
    in x and y and N x R in B and C."""
    es = 4 if wl.dtype == "f32" else 2
    if mimo:
        R = mimo
        if wl.layers > 1:
            per_layer = (2 * wl.batch * wl.D * wl.N * 4 + (2 * R + 1) * wl.batch * wl.D * es
                         + 2 * wl.batch * wl.N * R * es + wl.D * wl.N * 4)
            if trapezoid:   # lam, and the previous token's x and B rows
                per_layer += (R + 1) * wl.batch * wl.D * es + wl.batch * wl.N * R * es
            return per_layer * wl.layers
        return ((2 * R + 1 + (1 if trapezoid else 0)) * wl.batch * wl.L * wl.D * es
                + 2 * wl.batch * wl.L * wl.N * R * es + wl.D * wl.N * 4 + wl.batch * wl.D * wl.N * 4)
    if wl.layers > 1:  # decode: state read + write, token rows in and out, A, per layer
        per_layer = 2 * wl.batch * wl.D * wl.N * 4 + 3 * wl.batch * wl.D * es + 2 * wl.batch * wl.N * es + wl.D * wl.N * 4
        if trapezoid:
            per_layer += 2 * wl.batch * wl.D * es + wl.batch * wl.N * es
        return per_layer * wl.layers
    return ((4 if trapezoid else 3) * wl.batch * wl.L * wl.D * es + 2 * wl.batch * wl.L * wl.N * es
            + wl.D * wl.N * 4 + wl.batch * wl.D * wl.N * 4)


def read_traffic(workload: str, launches_per_step: int):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        m = re.match(r"\s*(\w+)\s*=\s*([0-9.eE+-]+|[0-9a-f]+)\s*$", line)
        if m:
            vals[m.group(1)] = m.group(2)
    kind = ("step" if workload.startswith("decode") else "prefill") + ("_mimo" if "_mimo" in workload else "")
    if vals.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(wl, inp, channels: int, scalar_a=None, complex_a=False, lam=None, mimo=0):
    """The fp64 oracle, as it stands, on a bounded sample: all tokens of `channels` channels
    (with `scalar_a`, the scaled-identity oracle on that A; with `complex_a`, the complex-state
    oracle on inp["A"]; with `lam`, the exponential-trapezoidal oracle).  Returns the report
    and the oracle's (y, h_final) on the sample, which the bench compares with its own outputs."""
    import numpy as np

    import oracle

    threads = min(16, len(os.sched_getaffinity(0)))
    x = inp["x"][:, :, :channels]
    dl = inp["delta"][:, :, :channels]
    A = inp["A"][:channels] if scalar_a is None else scalar_a[:channels]
    args = [np.ascontiguousarray(t.float().numpy(), dtype=np.float64) for t in (x, dl, A, inp["B"], inp["C"])]
    fn = oracle.prefill_complex if complex_a else oracle.prefill if scalar_a is None else oracle.prefill_scalar_a
    t0 = time.perf_counter()
    form = "complex" if complex_a else "diagonal" if scalar_a is None else "scalar"
    if mimo and lam is not None:
        lm = np.ascontiguousarray(lam[:, :, :channels].float().numpy(), dtype=np.float64)
        ref = oracle.prefill_mimo_trapezoid(args[0], args[1], lm, *args[2:], form=form, nthreads=threads)
    elif mimo:
        ref = oracle.prefill_mimo(*args, form=form, nthreads=threads)
    elif lam is not None:
        lm = np.ascontiguousarray(lam[:, :, :channels].float().numpy(), dtype=np.float64)
        ref = oracle.prefill_trapezoid(args[0], args[1], lm, *args[2:], form=form, nthreads=threads)
    else:
        ref = fn(*args, nthreads=threads)
    dt = time.perf_counter() - t0
    elems = wl.batch * wl.L * channels
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(line.split(":", 1)[1].strip() for line in fh if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    out = {"value": elems / dt, "unit": "elems/s", "cores": threads, "kind": "oracle",
           "sample": f"{wl.name}: batch {wl.batch}, all {wl.L} tokens, first {channels} of {wl.D} channels, "
                     f"N {wl.N}, fp64 ({dt:.1f} s on {threads} threads)",
           "host_cpu": cpu, "host_cpus": os.cpu_count(), "cpus_allowed": len(os.sched_getaffinity(0)),
           "threads": threads}
    return out, ref


def single_thread_rate():
    """The oracle on one thread over a bounded sample of the 4K workload (all 4096 tokens of
    its first 256 channels): elems/s of B*L*D."""
    import numpy as np

    import oracle
    import workloads

    wl = workloads.get("prefill_4k")
    inp = workloads.prefill_inputs(wl)
    ch = 256
    args = [np.ascontiguousarray(t.float().numpy(), dtype=np.float64)
            for t in (inp["x"][:, :, :ch], inp["delta"][:, :, :ch], inp["A"][:ch], inp["B"], inp["C"])]
    t0 = time.perf_counter()
    oracle.prefill(*args, nthreads=1)
    dt = time.perf_counter() - t0
    return {"value": wl.batch * wl.L * ch / dt, "unit": "elems/s", "threads": 1,
            "sample": f"prefill_4k: all {wl.L} tokens, first {ch} of {wl.D} channels ({dt:.2f} s)"}


def run_micro_scan(log):
    """The wavefront-level associative scan of (a, b) pairs over the 64 lanes of a wave, by DPP
    (libjscan_micro kind 11: 6 levels of a DPP-fed FMA and multiply on 8 independent chains),
    beside the FMA and the DPP-broadcast multiply it is built from, at 8 waves and 1 wave per
    SIMD.  Reports cycles per wave instruction and the combine's cost per (a, b) element in FMA
    slots, to set against the sequential scan's 7.05 slots for a whole state element."""
    import torch

    from mamba_selective_scan_03_amd import micro

    cus = 256
    out = {"gpu": torch.cuda.get_device_name(0), "rocm": torch.version.hip}
    ms, clk, ticks = micro.valu(0, 100000, 2048, 256)
    hz = clk / (ticks / 100e6)
    out["shader_clock_GHz"] = round(hz / 1e9, 3)

    def cycles_per_instr(kind, waves_per_simd, iters, per_trip):
        ms, _, _ = micro.valu(kind, iters, cus * waves_per_simd, 256)
        return ms * 1e-3 * hz / (waves_per_simd * iters * per_trip)

    rows = {}
    for kind, name, per_trip in ((0, "fma", 16), (4, "mul_dpp_bcast", 16), (11, "wave_scan_level_dpp", 96)):
        rows[name] = {f"cycles_per_instr_{w}w": round(cycles_per_instr(kind, w, iters // per_trip * 16, per_trip), 3)
                      for w, iters in ((8, 20000), (1, 80000))}
        log(f"micro {name}: {rows[name]}")
    out["valu_cycles_per_wave_instruction"] = rows
    c_fma = rows["fma"]["cycles_per_instr_8w"]
    c_lvl = rows["wave_scan_level_dpp"]["cycles_per_instr_8w"]
    out["derived"] = {
        "scan_levels": 6,
        "instructions_per_element": 12,
        "combine_cost_in_fma_slots_per_element": round(12 * c_lvl / c_fma, 2),
        "sequential_state_element_fma_slots": 7.05,
    }
    return out


def run_micro(log):
    """The microbenchmarks of libjscan_micro: vector-ALU issue rates (FMA, exponential, their
    mix, DPP and permlane forms) at 8 waves and at 1 wave per SIMD, matrix cores beside the
    vector ALU, the matrix core's rounding of a*b + c, LDS read bandwidth and HBM streams.
    Returns one dict of measured and derived rates."""
    import torch

    from mamba_selective_scan_03_amd import micro

    cus, simds = 256, 1024
    out = {"gpu": torch.cuda.get_device_name(0), "rocm": torch.version.hip}
    # shader clock from the FMA loop: clocks over 100 MHz reference ticks
    ms, clk, ticks = micro.valu(0, 100000, 2048, 256)
    ghz = clk / (ticks / 100e6) / 1e9
    out["shader_clock_GHz"] = round(ghz, 3)
    hz = ghz * 1e9

    def cycles_per_instr(kind, waves_per_simd, iters, per_trip=16):
        # work-groups of 4 waves, one per SIMD of a CU; waves_per_simd work-groups per CU
        blocks = cus * waves_per_simd
        ms, _, _ = micro.valu(kind, iters, blocks, 256)
        instr_per_simd = waves_per_simd * iters * per_trip
        return ms * 1e-3 * hz / instr_per_simd

    # where the waves of a 256-work-group launch land: at most this many share a SIMD
    out["max_waves_per_simd_1w"] = micro.valu(0, 1000, cus, 256, placement=True)[3]
    out["max_waves_per_simd_2w"] = micro.valu(0, 1000, 2 * cus, 256, placement=True)[3]
    valu = {}
    for kind, name in micro.VALU_KINDS.items():
        row = {}
        for w, iters in ((8, 20000), (4, 40000), (2, 80000), (1, 80000)):
            if w in (2, 4) and kind not in (0, 1, 10):
                continue
            row[f"cycles_per_instr_{w}w"] = round(cycles_per_instr(kind, w, iters), 3)
        valu[name] = row
        log(f"micro valu {name}: {row}")
    out["valu_cycles_per_wave_instruction"] = valu
    # the scan's token body for a lane of two states: cycles per token per wave
    body = {}
    for kind, name in ((8, "sgpr_bc"), (9, "dpp_bc")):
        row = {}
        for w in (1, 2, 4, 8):
            row[f"cycles_per_token_{w}w"] = round(cycles_per_instr(kind, w, 160000 // w, per_trip=4), 2)
        body[name] = row
        log(f"micro scan body {name}: {row}")
    out["scan_token_body_cycles"] = body
    c_fma = valu["fma"]["cycles_per_instr_8w"]
    c_exp = valu["exp"]["cycles_per_instr_8w"]
    mix = valu["exp8+fma8"]["cycles_per_instr_8w"] * 16
    pair = valu["mul+exp pairs"]["cycles_per_instr_8w"] * 16 / 8
    swap = (valu["permlane32_swap+max"]["cycles_per_instr_8w"] * 16 - 8 * c_fma) / 8
    out["derived"] = {
        "fma_lane_ops_per_CU_clock": round(4 * 64 / c_fma, 2),
        "exp_lane_ops_per_CU_clock": round(4 * 64 / c_exp, 2),
        "exp_cost_in_fma_slots": round(c_exp / c_fma, 3),
        "exp8_fma8_trip_cycles": round(mix, 1),
        "exp8_fma8_if_serial": round(8 * c_exp + 8 * c_fma, 1),
        "exp8_fma8_if_overlapped": round(max(8 * c_exp, 8 * c_fma), 1),
        "mul_exp_pair_cost_in_fma_slots": round(pair / c_fma, 3),
        "permlane32_swap_cost_in_fma_slots": round(swap / c_fma, 3),
        "mul_dpp_cost_in_fma_slots": round(valu["mul_dpp_bcast"]["cycles_per_instr_8w"] / c_fma, 3),
        "valu_lane_slots_per_s": round(cus * 4 * 64 * hz / c_fma, -9),
    }

    # matrix cores beside the vector ALU: 4 waves per SIMD, then one wave per SIMD
    mf = {}
    for label, blocks, threads, iters in (("4w", 1024, 256, 16000), ("1w", 256, 256, 64000)):
        waves = blocks * threads // 64 / simds
        t = [micro.mfma_valu(m, iters, blocks, threads) for m in (0, 1, 2, 3, 4)]
        mf[label] = {"mfma_only_ms": round(t[0], 3), "valu_only_ms": round(t[1], 3), "both_ms": round(t[2], 3),
                     "overlap": round((t[0] + t[1] - t[2]) / min(t[0], t[1]), 3),
                     "mfma_16x16x4_f32_cycles": round(t[0] * 1e-3 * hz / (waves * iters * 4), 2),
                     "fma_cycles": round(t[1] * 1e-3 * hz / (waves * iters * 32), 2),
                     "bf16_mfma_only_ms": round(t[3], 3), "bf16_both_ms": round(t[4], 3),
                     "bf16_overlap": round((t[3] + t[1] - t[4]) / min(t[3], t[1]), 3),
                     "mfma_16x16x32_bf16_cycles": round(t[3] * 1e-3 * hz / (waves * iters * 4), 2)}
    out["mfma_beside_valu"] = mf
    log(f"micro mfma beside valu: {mf}")

    g = torch.Generator().manual_seed(0)
    rnd = {}
    for variant, name in ((0, "4x4x1_16b"), (1, "16x16x4_onehot")):
        a = torch.randn(64, generator=g)
        b = torch.randn(64, generator=g)
        c = torch.randn(256, generator=g) * 4
        if variant == 1:
            # A[i][k] (lane i + 16 k) nonzero only for k = i % 4: one product per output
            lane = torch.arange(64)
            a = torch.where(lane // 16 == (lane % 16) % 4, a, torch.zeros(()))
        d1, d2 = micro.mfma_rounding(variant, a.cuda(), b.cuda(), c.cuda())
        diff = int((d1.view(torch.int32) != d2.view(torch.int32)).sum())
        rel = float(((d1 - d2).abs() / d2.abs().clamp_min(1e-30)).max())
        rnd[name] = {"values": 256, "bitwise_differences": diff, "max_rel_diff": rel}
    out["mfma_f32_vs_fmaf"] = rnd
    log(f"micro mfma rounding: {rnd}")

    iters = 20000
    lds = {}
    for unique in (64, 32, 16):
        ms = micro.lds(iters, 2048, 256, unique)
        # bytes the lanes asked for, and wave instructions per CU clock
        lds[f"unique{unique}"] = {"requested_bytes_per_CU_clock": round(2048 * 256 * iters * 128 / (ms * 1e-3 * hz) / cus, 1),
                                  "b128_reads_per_CU_clock": round(2048 * 4 * iters * 8 / (ms * 1e-3 * hz) / cus, 3)}
    out["lds_read"] = lds
    log(f"micro lds: {lds}")

    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    hbm = {}
    for kind, name in ((0, "read"), (1, "write"), (2, "copy")):
        for nt in (False, True):
            best = None
            for blocks in (1024, 2048, 4096, 8192):
                ms = micro.hbm(kind, nt, src, dst, nbytes, blocks, 10) / 10
                moved = nbytes * (2 if kind == 2 else 1)
                gbps = moved / (ms * 1e-3) / 1e9
                if best is None or gbps > best[0]:
                    best = (gbps, blocks)
            hbm[f"{name}{'_nt' if nt else ''}"] = {"GBps": round(best[0], 1), "blocks": best[1]}
    out["hbm_1GiB_streams"] = hbm
    log(f"micro hbm: {hbm}")
    return out


def trace_summary(directory: str, warmup: int) -> str:
    """Per-kernel durations from rocprofv3 --kernel-trace CSV files, in launch order, leaving out
    each kernel's first `warmup` launches; one line per kernel (microseconds)."""
    import csv
    import glob
    import statistics
    rows = []
    for path in sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)):
        with open(path, newline="") as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    by_kernel = {}
    for r in rows:
        by_kernel.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = []
    for name, us in by_kernel.items():
        kept = us[warmup:] if len(us) > warmup else us
        # the bench also makes short launches of its own (checks on a few tokens): leave out
        # those under a quarter of the median
        med = statistics.median(kept)
        short = [u for u in kept if u < med / 4]
        kept = [u for u in kept if u >= med / 4]
        out.append(f"{name}\n    launches {len(us)}, after the first {len(us) - len(kept) - len(short)}"
                   f"{f' (and {len(short)} short ones)' if short else ''}: median "
                   f"{statistics.median(kept):.1f} us, mean {statistics.fmean(kept):.1f}, min {min(kept):.1f}, "
                   f"max {max(kept):.1f}")
    return "\n".join(out)


def counter_summary(args, fetch_dir: str, write_dir: str) -> str:
    """HBM traffic of the dominant kernel of a workload and mode from two rocprofv3 --pmc runs
    (FETCH_SIZE in fetch_dir, WRITE_SIZE in write_dir), per launch (every dispatch of the kernel
    is counted: mean, and the spread over dispatches), scaled by what the counters read for a
    plain device-to-device copy of 1 GiB (profiles/counters_copy_calibration.txt)."""
    import csv
    import glob
    import statistics
    import workloads
    wl = workloads.get(args.workload)
    decode = wl.layers > 1
    name = ("jscan::step_mimo_kernel<" if args.mimo else "jscan::step_kernel<") if decode else \
        ("jscan::prefill_mimo_rows_kernel<" if args.mimo else "jscan::prefill_rows_kernel<")
    cal = {}
    for line in open(os.path.join(ROOT, "profiles", "counters_copy_calibration.txt")):
        m = re.match(r"\s*(\w+)\s*=\s*([0-9.eE+-]+)\s*$", line)
        if m:
            cal[m.group(1)] = float(m.group(2))
    fetch_scale = (1 << 20) / cal["copy_fetch_KiB_per_GiB"]
    write_scale = (1 << 20) / cal["copy_write_KiB_per_GiB"]

    def per_dispatch(directory, counter):
        # the workload's launches are the kernel's long ones (the bench also makes short
        # launches of its own, e.g. the bit-exactness check on a few tokens)
        vals, dur = {}, {}
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            with open(path, newline="") as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter and r["Kernel_Name"].startswith("void " + name):
                        key = (path, r["Dispatch_Id"])
                        vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
                        dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        top = max(dur.values(), default=0)
        return [v for k, v in vals.items() if dur[k] >= top / 2]
    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    if not fetch or not write:
        return f"no dispatches of {name} in {fetch_dir} / {write_dir}"
    alg = algorithmic_bytes(wl, args.trapezoid, args.mimo)
    if args.scalar_a:
        alg -= (wl.D * wl.N - wl.D) * 4 * max(wl.layers, 1)
    launches = wl.layers if decode else 1
    rd = statistics.fmean(fetch) * 1024 * fetch_scale
    wr = statistics.fmean(write) * 1024 * write_scale
    kind = ("step" if decode else "prefill") + ("_mimo" if args.mimo else "")
    lines = [
        f"kernel = {name}...>",
        f"fetch_scale = {fetch_scale:.4f}",
        f"write_scale = {write_scale:.4f}",
        f"dispatches_fetch = {len(fetch)}",
        f"dispatches_write = {len(write)}",
        f"FETCH_SIZE_KiB_per_launch = {statistics.fmean(fetch):.6g}",
        f"FETCH_SIZE_KiB_per_launch_min_median_max = {min(fetch):.6g} {statistics.median(fetch):.6g} {max(fetch):.6g}",
        f"WRITE_SIZE_KiB_per_launch = {statistics.fmean(write):.6g}",
        f"WRITE_SIZE_KiB_per_launch_min_median_max = {min(write):.6g} {statistics.median(write):.6g} {max(write):.6g}",
        f"hbm_read_bytes_per_launch = {rd:.6g}",
        f"hbm_write_bytes_per_launch = {wr:.6g}",
        f"hbm_bytes_per_launch = {rd + wr:.6g}",
        f"algorithmic_bytes_per_launch = {alg // launches}",
        f"traffic_over_algorithmic = {(rd + wr) / (alg / launches):.4f}",
        f"kernel_source_hash = {kernel_source_hash(kind)}",
    ]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps before the timed ones (default: at least 5, and as many more as fill one "
                         "second: short steps run slower until the GPU has been busy for about that long)")
    ap.add_argument("--workload", default="prefill_64k",
                    choices=["prefill_64k", "prefill_4k", "prefill_256k", "decode_256x28", "tiny_fp32",
                             "prefill_64k_tp8", "prefill_16x4k"])
    ap.add_argument("--producer", action="store_true",
                    help="prefill workloads: compute delta, B and C from x with jscan_ssm_inputs (synthetic weights, "
                         "rank 256) inside each step, then scan")
    ap.add_argument("--fused", action="store_true",
                    help="with --producer: compute delta inside the scan (jscan_prefill_fused) instead of storing it")
    ap.add_argument("--chunked", action="store_true",
                    help="prefill through the time-parallel jscan_prefill_chunked (automatic segments) instead of "
                         "the token-by-token jscan_prefill")
    ap.add_argument("--scalar-a", action="store_true",
                    help="A is a scaled identity, one value per channel (the Mamba-2 form): "
                         "jscan_prefill_scalar_a / jscan_step_scalar_a")
    ap.add_argument("--complex-a", action="store_true",
                    help="complex-valued state, pairs of the 16 states as 8 complex states (the Mamba-3 form): "
                         "jscan_prefill_complex / jscan_step_complex")
    ap.add_argument("--trapezoid", action="store_true",
                    help="the exponential-trapezoidal rule (the Mamba-3 discretisation), with the diagonal A or "
                         "with --scalar-a / --complex-a: jscan_prefill_trapezoid / jscan_step_trapezoid")
    ap.add_argument("--mimo", type=int, default=0, metavar="R", choices=[0, 1, 2, 4, 8],
                    help="the MIMO scan with R inputs and outputs per channel (B and C N x R), with the diagonal A "
                         "or with --scalar-a / --complex-a: jscan_prefill_mimo / jscan_step_mimo")
    ap.add_argument("--cpu-channels", type=int, default=8192,
                    help="oracle sample: all tokens of the first CPU_CHANNELS channels (default: every channel "
                         "of the 64K workload, a few seconds on 16 cores; 0 = skip)")
    ap.add_argument("--micro-scan", action="store_true",
                    help="time the wavefront-level (a, b) scan combine by DPP against the FMA (no bench line)")
    ap.add_argument("--micro", action="store_true",
                    help="instead of the scan, run the microbenchmarks (vector ALU, matrix cores, LDS, HBM) and print "
                         "their rates as one JSON line")
    ap.add_argument("--cpu-single-thread", action=argparse.BooleanOptionalAction, default=True,
                    help="also time the oracle on one thread over a sample of the 4K workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the scan, time a plain device-to-device copy of MIB mebibytes (the reference "
                         "kernel for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--counter-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="instead of the scan, summarise two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of "
                         "this workload and mode: the dominant kernel's HBM bytes per launch, scaled by the copy "
                         "calibration in profiles/counters_copy_calibration.txt, against its algorithmic bytes")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="instead of the scan, summarise the rocprofv3 kernel trace(s) in DIR (*kernel_trace.csv): "
                         "per kernel, the launches after the first WARMUP, their median, mean, min and max")
    args = ap.parse_args()

    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.warmup or 0))
        return
    if args.counter_summary:
        print(counter_summary(args, *args.counter_summary))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the benchmark runs on one GPU; sharding the scan over several GPUs is described in the "
              "design notes, not implemented. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    import mamba_selective_scan_03_amd as jscan
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.micro_scan:
        torch.cuda.set_device(dev)
        print(json.dumps({"micro_scan": run_micro_scan(lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))}),
              flush=True)
        return
    if args.micro:
        torch.cuda.set_device(dev)
        print(json.dumps({"micro": run_micro(lambda *a: print("[bench]", *a, file=sys.stderr, flush=True))}),
              flush=True)
        return
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup or 5):
            dst.copy_(src)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / args.steps
        print(json.dumps({"calibration": "copy", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
                          "ms_per_launch": ms, "GBps": 2 * n * 4 / ms / 1e6}), flush=True)
        return
    wl = workloads.get(args.workload)
    if (args.scalar_a or args.complex_a or args.trapezoid or args.mimo) and (args.producer or args.chunked):
        print("bench.py: --scalar-a, --complex-a, --trapezoid and --mimo run the plain prefill or decode step only",
              file=sys.stderr)
        sys.exit(2)
    if args.scalar_a and args.complex_a:
        print("bench.py: choose one of --scalar-a and --complex-a", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(dev)
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)  # noqa: E731

    form = "scalar" if args.scalar_a else "complex" if args.complex_a else "diagonal"
    t0 = time.perf_counter()
    if wl.layers > 1:
        layers = []
        for layer in range(wl.layers):
            # the trapezoidal rule's step is token 1, with token 0 as its previous token
            token = 1 if args.trapezoid else 0
            if args.mimo:
                inp = workloads.decode_layer_mimo_inputs(wl, layer, args.mimo, token=token)
                prev = workloads.decode_layer_mimo_inputs(wl, layer, args.mimo, token=0) if args.trapezoid else None
                inp["lam"] = workloads.decode_layer_inputs(wl, layer, token=token)["lam"]
            else:
                inp = workloads.decode_layer_inputs(wl, layer, token=token)
                prev = workloads.decode_layer_inputs(wl, layer, token=0) if args.trapezoid else None
            if args.trapezoid:
                inp["x_prev"], inp["B_prev"] = prev["x"], prev["B"]
            else:
                inp.pop("lam")
            if args.scalar_a:
                inp["A"] = workloads.draw_scalar_a(wl, layer=layer)
            if args.complex_a:
                inp["A"] = workloads.draw_complex_a(wl, layer=layer)
            layers.append({k: v.to(dev) for k, v in inp.items()})
            layers[-1]["h"] = layers[-1].pop("h0")

        for L_ in layers:
            L_["y"] = torch.empty_like(L_["x"])
        step_fn = jscan.step_scalar_a if args.scalar_a else jscan.step_complex if args.complex_a else jscan.step

        def token_step():
            for L_ in layers:
                if args.mimo and args.trapezoid:
                    jscan.step_mimo_trapezoid(L_["h"], L_["x_prev"], L_["B_prev"], L_["x"], L_["delta"], L_["lam"],
                                              L_["A"], L_["B"], L_["C"], form=form, y_t=L_["y"])
                elif args.mimo:
                    jscan.step_mimo(L_["h"], L_["x"], L_["delta"], L_["A"], L_["B"], L_["C"], form=form, y_t=L_["y"])
                elif args.trapezoid:
                    jscan.step_trapezoid(L_["h"], L_["x_prev"], L_["B_prev"], L_["x"], L_["delta"], L_["lam"],
                                         L_["A"], L_["B"], L_["C"], form=form, y_t=L_["y"])
                else:
                    step_fn(L_["h"], L_["x"], L_["delta"], L_["A"], L_["B"], L_["C"], y_t=L_["y"])

        # One token step is 28 short launches; a captured HIP graph replays them without the
        # host launch overhead of 28 separate calls.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            token_step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            token_step()

        def one_step():
            graph.replay()
        launches = wl.layers
        host_inp = None
    else:
        host_inp = workloads.mimo_inputs(wl, args.mimo) if args.mimo else workloads.prefill_inputs(wl)
        d = {k: v.to(dev) for k, v in host_inp.items()}
        y = torch.empty_like(d["x"])
        h = torch.empty((wl.batch, wl.D, wl.N), dtype=torch.float32, device=dev)

        if args.producer:
            if wl.dtype != "bf16":
                print("bench.py: --producer needs a bf16 workload", file=sys.stderr)
                sys.exit(2)
            pw = {k: v.to(dev) for k, v in workloads.producer_weights(wl.D, PRODUCER_RANK).items()}
            d["delta"] = torch.empty_like(d["x"])
            d["B"] = torch.empty_like(d["B"])
            d["C"] = torch.empty_like(d["C"])
            d_low = torch.empty((wl.batch, wl.L, PRODUCER_RANK), dtype=torch.bfloat16, device=dev)

            if args.fused:
                def produce():
                    jscan.ssm_inputs(d["x"], pw["w_x"], pw["g_d"], pw["g_b"], pw["g_c"], pw["w_dt"], pw["b_dt"],
                                     B=d["B"], C=d["C"], delta_low=d_low, skip_delta=True)

                def scan():
                    jscan.prefill_fused(d["x"], d_low, pw["w_dt"], pw["b_dt"], d["A"], d["B"], d["C"], y=y, h_final=h)
            else:
                def produce():
                    jscan.ssm_inputs(d["x"], pw["w_x"], pw["g_d"], pw["g_b"], pw["g_c"], pw["w_dt"], pw["b_dt"],
                                     delta=d["delta"], B=d["B"], C=d["C"], delta_low=d_low)

                def scan():
                    jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y, h_final=h)

            def one_step():
                produce()
                scan()
            launches = 2 if args.fused else 3
        elif args.chunked:
            ws_bytes = jscan.chunked_workspace_bytes(wl.batch, wl.L, wl.D)
            ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
            log(f"time-parallel prefill: {ws_bytes} bytes of workspace")

            def one_step():
                jscan.prefill_chunked(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y, h_final=h, workspace=ws)
            launches = 3 if ws_bytes > 0 else 1
        elif args.mimo:
            if args.scalar_a:
                host_a = workloads.draw_scalar_a(wl)
                d["A"] = host_a.to(dev)
            elif args.complex_a:
                host_inp["A"] = workloads.draw_complex_a(wl)
                d["A"] = host_inp["A"].to(dev)
            if args.trapezoid:
                host_inp["lam"] = workloads.lam_inputs(wl)
                d["lam"] = host_inp["lam"].to(dev)

                def one_step():
                    jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form, y=y,
                                                 h_final=h)
            else:
                def one_step():
                    jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], form=form, y=y, h_final=h)
            launches = 1
        elif args.trapezoid:
            host_inp["lam"] = workloads.lam_inputs(wl)
            d["lam"] = host_inp["lam"].to(dev)
            if args.scalar_a:
                host_a = workloads.draw_scalar_a(wl)
                d["A"] = host_a.to(dev)
            elif args.complex_a:
                host_inp["A"] = workloads.draw_complex_a(wl)
                d["A"] = host_inp["A"].to(dev)

            def one_step():
                jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form, y=y,
                                        h_final=h)
            launches = 1
        elif args.complex_a:
            host_inp["A"] = workloads.draw_complex_a(wl)
            d["A"] = host_inp["A"].to(dev)

            def one_step():
                jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y, h_final=h)
            launches = 1
        elif args.scalar_a:
            host_a = workloads.draw_scalar_a(wl)
            d["a"] = host_a.to(dev)

            def one_step():
                jscan.prefill_scalar_a(d["x"], d["delta"], d["a"], d["B"], d["C"], y=y, h_final=h)
            launches = 1
        else:
            def one_step():
                jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y, h_final=h)
            launches = 1
    torch.cuda.synchronize()
    log(f"inputs for {wl.name} resident in HBM ({time.perf_counter() - t0:.1f} s)")

    warmup = args.warmup if args.warmup is not None else 5
    for _ in range(warmup):
        one_step()
    torch.cuda.synchronize()
    if args.warmup is None:
        # Short steps measured right after start run up to 10% slower than after a second of
        # work (prefill_64k_tp8 through the time-parallel path: 0.362 ms after 10 warm-up steps,
        # 0.328 ms after 3000); the default warm-up therefore lasts at least one second.
        w0 = time.perf_counter()
        while time.perf_counter() - w0 < 1.0:
            for _ in range(10):
                one_step()
            warmup += 10
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        one_step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    log(f"{args.steps} steps: {ms_total:.3f} ms by HIP events, {wall * 1e3:.3f} ms wall")

    # Per-step times, taken after the timed region: median and minimum.  A workload whose bytes
    # fit in the 256 MB last-level cache is timed cold, with 512 MiB of scratch written between
    # steps (outside the events).
    cold = algorithmic_bytes(wl, args.trapezoid, args.mimo) < (1 << 30)
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if cold else None
    marks = []
    for _ in range(min(args.steps, 50)):
        if scratch is not None:
            scratch.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        one_step()
        b.record(stream)
        marks.append((a, b))
    torch.cuda.synchronize()
    per_step = sorted(a.elapsed_time(b) for a, b in marks)
    del scratch

    elems = wl.elems
    value = elems / (ms_step * 1e-3)
    alg_bytes = algorithmic_bytes(wl, args.trapezoid, args.mimo)
    if args.scalar_a:   # A is [D] instead of [D, N]
        alg_bytes -= (wl.D * wl.N - wl.D) * 4 * max(wl.layers, 1)
    gbps = alg_bytes / (ms_step * 1e-3) / 1e9
    per_launch_ms = ms_step / launches
    producer_info = None
    if args.producer:
        # time the two stages alone too (same stream, HIP events), for the per-stage rooflines
        def timed(fn, n):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(n):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / n
        p_ms, s_ms = timed(produce, args.steps), timed(scan, args.steps)
        tokens = wl.batch * wl.L
        flops = 2 * tokens * wl.D * (PRODUCER_RANK + 2 * wl.N)
        hbm = tokens * wl.D * 2 + tokens * (PRODUCER_RANK + 2 * wl.N) * 2
        if not args.fused:   # the delta projection runs in the producer, not inside the scan
            flops += 2 * tokens * PRODUCER_RANK * wl.D
            hbm += tokens * wl.D * 2 + tokens * (PRODUCER_RANK + 2 * wl.N) * 2
        producer_info = {"ms": round(p_ms, 4), "scan_ms": round(s_ms, 4), "rank": PRODUCER_RANK,
                         "mfma_TFLOPs": round(flops / (p_ms * 1e-3) / 1e12, 1), "mfma_peak_TFLOPs": BF16_MFMA_PEAK_TFLOPS,
                         "mfma_frac": round(flops / (p_ms * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                         "hbm_GBps": round(hbm / (p_ms * 1e-3) / 1e9, 1),
                         "hbm_frac": round(hbm / (p_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        log(f"producer {p_ms:.3f} ms, scan {s_ms:.3f} ms")
        # the scan kernel stays the dominant kernel for the roofline object below
        per_launch_ms = s_ms
    if args.chunked:
        # three launches per step (segment summaries, carry, rescan): the line reports the
        # whole pass against the one-pass ALU bound
        per_launch_ms = ms_step
    # The metric's roofline is HBM: algorithmic bytes of one launch of the dominant kernel over
    # its average launch time (HIP events on the stream the kernels run on).  For the prefill the
    # binding resource is the vector ALU, so its issue-bound fraction is reported beside it.
    hbm_achieved = alg_bytes / launches / (per_launch_ms * 1e-3) / 1e9
    if args.producer or args.chunked:
        hbm_achieved = alg_bytes / (per_launch_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(hbm_achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(hbm_achieved / HBM_PEAK_GBPS, 4)}
    roofline["traffic"] = None if (args.chunked or args.producer) else read_traffic(
        wl.name + ("_scalar_a" if args.scalar_a else "_complex_a" if args.complex_a else "")
        + ("_trapezoid" if args.trapezoid else "") + (f"_mimo{args.mimo}" if args.mimo else ""), launches)
    roofline_alu = None
    if wl.layers == 1:
        state_elems = elems * wl.N
        slots, flops = ((SCALAR_A_SLOTS, SCALAR_A_FLOPS) if args.scalar_a else
                        (COMPLEX_A_SLOTS, COMPLEX_A_FLOPS) if args.complex_a else
                        (SLOTS_PER_STATE_ELEM, FLOPS_PER_STATE_ELEM))
        if args.trapezoid:
            slots, flops = slots + TRAP_SLOTS, flops + TRAP_FLOPS
        if args.mimo:
            slots, flops = mimo_cost(form, args.mimo)
            if args.trapezoid:
                slots, flops = slots + args.mimo, flops + 2 * args.mimo
        achieved_tf = state_elems * flops / (per_launch_ms * 1e-3) / 1e12
        peak_tf = VALU_SLOTS_PER_S / slots * flops / 1e12
        roofline_alu = {"bound": "alu", "achieved": round(achieved_tf, 2), "peak": round(peak_tf, 2),
                        "unit": "TFLOP/s", "frac": round(achieved_tf / peak_tf, 4), "slots_per_state_elem": slots,
                        "hbm_frac_at_this_bound": round(alg_bytes * VALU_SLOTS_PER_S / slots / state_elems
                                                        / 1e9 / HBM_PEAK_GBPS, 4)}

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "L": wl.L, "D": wl.D, "N": wl.N,
                   "layers": wl.layers, "io_dtype": wl.dtype, "state_dtype": "f32",
                   "A": "scaled_identity" if args.scalar_a else "complex_pairs" if args.complex_a else "diagonal",
                   "discretisation": "exponential-trapezoidal" if args.trapezoid else "euler",
                   "mimo_rank": args.mimo or 1,
                   "path": ("producer+fused-scan" if args.fused else "producer+scan") if args.producer
                   else ("time-parallel" if args.chunked else "sequential")},
        "step_ms_median": round(per_step[len(per_step) // 2], 4),
        "step_ms_min": round(per_step[0], 4),
        "step_timing": "cold: 512 MiB written between steps" if cold else "back to back",
        "hbm_GBps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_step": alg_bytes,
        "roofline": roofline,
        "roofline_alu": roofline_alu,
    }
    if producer_info is not None:
        out["producer"] = producer_info
    out.update(run_info(torch, ("step" if wl.layers > 1 else "prefill") + ("_mimo" if args.mimo else "")))
    if host_inp is not None and args.cpu_channels > 0 and wl.layers == 1:
        ch = min(args.cpu_channels, wl.D)
        out["cpu_baseline"], ref = cpu_baseline(wl, host_inp, ch, host_a if args.scalar_a else None,
                                                complex_a=args.complex_a,
                                                lam=host_inp.get("lam") if args.trapezoid else None, mimo=args.mimo)
        log(f"oracle sample: {out['cpu_baseline']['sample']}")
        if args.cpu_single_thread:
            out["cpu_baseline"]["single_thread"] = single_thread_rate()
        if not args.producer:
            # the timed run's own outputs (last step) against the oracle on the sampled channels
            import numpy as np

            y_ref, h_ref = ref
            y_got = y[..., :ch, :] if args.mimo else y[..., :ch]
            err_y = float(np.max(np.abs(y_got.double().cpu().numpy() - y_ref))) / float(np.max(np.abs(y_ref)))
            err_h = float(np.max(np.abs(h[:, :ch].double().cpu().numpy() - h_ref))) / float(np.max(np.abs(h_ref)))
            out["parity_max_rel"] = {"y": float(f"{err_y:.3e}"), "h_final": float(f"{err_h:.3e}"),
                                     "tol": 1e-4 if wl.dtype == "f32" else 2e-2,
                                     "channels": f"first {ch} of {wl.D}, all tokens"}
    if wl.layers == 1 and not (args.producer or args.chunked or args.mimo or args.trapezoid or args.scalar_a
                               or args.complex_a):
        out["bitexact_ok"] = bitexact_check(jscan, d, wl)
    print(json.dumps(out), flush=True)


def run_info(torch, kind: str):
    """GPU, ROCm and source identification for the report line; `kind` names the timed
    kernel's sources (a key of KERNEL_SOURCES)."""
    props = torch.cuda.get_device_properties(0)
    info = {"gpu": torch.cuda.get_device_name(0), "gpu_arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": torch.version.hip, "torch": torch.__version__}
    sha = None
    try:
        import subprocess

        sha = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True, text=True,
                             timeout=10).stdout.strip() or None
    except (OSError, subprocess.SubprocessError):
        pass
    info["git_sha"] = sha   # None where the tree was copied without its history
    info["kernel_source_hash"] = kernel_source_hash(kind)
    return info


def bitexact_check(jscan, d, wl, tokens: int = 256):
    """The first `tokens` tokens of the workload through jscan_prefill and through as many
    jscan_step calls from the zero state: the two final states must be equal bit for bit."""
    import torch

    x, dl, B, C = (d[k][:, :tokens].contiguous() for k in ("x", "delta", "B", "C"))
    _, h_pre = jscan.prefill(x, dl, d["A"], B, C)
    h = torch.zeros_like(h_pre)
    y_t = torch.empty((wl.batch, wl.D), dtype=x.dtype, device=x.device)
    for t in range(tokens):
        jscan.step(h, x[:, t], dl[:, t], d["A"], B[:, t], C[:, t], y_t=y_t)
    torch.cuda.synchronize()
    return bool(torch.equal(h.view(torch.int32), h_pre.view(torch.int32)))


if __name__ == "__main__":
    main()

#!/usr/bin/env python3
"""Benchmark of the selective-scan hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill_64k]

One step is one full pass of the hot path over one batch: a jscan_prefill of the whole
sequence (prefill workloads) or one decode token through all layers (decode workload).
Inputs are generated once, moved to HBM, and stay resident; the timed region holds only
the library's kernels, bracketed by stream synchronisation and timed with HIP events on
the stream the kernels run on.  Prints exactly one JSON line.

The roofline of the prefill kernel is its VALU issue rate, not HBM: each state element
needs 5 fp32 instructions (the exponent product, the base-2 exponential, the input
product and two fused multiply-adds), and the exponential issues at half rate, so
6 issue slots per element is the floor.  The chip issues 256 CUs x 4 SIMDs x 16 lanes x
2.4 GHz = 3.93e13 lane-slots/s, hence at most 6.55e12 state elements/s.  In flops the
five instructions are 7 operations (each FMA counts 2), so the same bound reads
45.9 TFLOP/s.  HBM traffic (about 6 bytes per B*L*D element in bf16) is reported beside
it as GB/s and as a fraction of 8 TB/s.

With --scalar-a (A a scaled identity, one value per channel: the Mamba-2 form) the decay is
shared by a channel's 16 states, so a state element needs only the input product and two
fused multiply-adds (3 slots) plus a sixteenth of the decay's product and exponential
(3/16): 3.1875 slots and 5.125 flops per element, a bound of 63.2 TFLOP/s.  With --complex-a
(the complex-valued state of the Mamba-3 form) one complex state, two elements, takes 19
slots and 21 flops per token (decay, rotation by a hardware sine and cosine, complex update,
output): 9.5 slots and 10.5 flops per element, a bound of 43.4 TFLOP/s.  --trapezoid (the
exponential-trapezoidal rule of Mamba-3, with any of the three forms of A) adds one fused
multiply-add per element, the previous token's input taken in before the decay: one slot and
two flops more than the form's own count, and lam [B, L, D] to the bytes read.  --mimo R (R
inputs and outputs per channel, B and C N x R: the MIMO scan of Mamba-3) makes the input term a
rank-R sum (one product and R - 1 fused multiply-adds) and the output R fused multiply-adds per
element: 2R + 4 slots and 4R + 3 flops for the diagonal A (12 and 19 at R = 4), 2R + 1 + 3/16
and 4R + 1 + 2/16 for the scaled identity, (15 + 4R) / 2 and (8R + 13) / 2 for the complex state;
x and y grow R-fold in bytes.  --mimo R --trapezoid (both Mamba-3 changes) adds the left end
point's R fused multiply-adds per element (R slots, 2R flops) and lam to the bytes.
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
VALU_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9      # fp32 lane-instructions per second (no packed math)
SLOTS_PER_STATE_ELEM = 6                      # mul, exp (2 slots), mul, fma, fma
FLOPS_PER_STATE_ELEM = 7                      # mul 1 + exp 1 + mul 1 + fma 2 + fma 2
PEAK_STATE_ELEMS = VALU_SLOTS_PER_S / SLOTS_PER_STATE_ELEM
SCALAR_A_SLOTS = 3 + 3 / 16                   # mul, fma, fma; decay (mul + exp) once per 16 states
SCALAR_A_FLOPS = 5 + 2 / 16
# complex state, per real component (half a complex state): decay mul + exp (3), angle mul +
# fract (2), cos and sin (4), r cos and r sin (2), two input products (2), four fma (4), y (2)
COMPLEX_A_SLOTS = 19 / 2
COMPLEX_A_FLOPS = 21 / 2
TRAP_SLOTS, TRAP_FLOPS = 1, 2                 # the left end point's fma, on top of the form's count


def mimo_cost(form: str, R: int):
    """(issue slots, flops) per state element of the rank-R scan; R = 1 gives the single-input counts."""
    if form == "scalar":
        return 2 * R + 1 + 3 / 16, 4 * R + 1 + 2 / 16
    if form == "complex":
        return (15 + 4 * R) / 2, (8 * R + 13) / 2
    return 2 * R + 4, 4 * R + 3
KERNEL_SOURCES = {
    "prefill": ["scan_update.h", "mfma_common.h", "prefill_rows_kernel.h"],
    "step": ["scan_update.h", "step_kernel.h"],
    "prefill_mimo": ["scan_update.h", "mfma_common.h", "prefill_rows_kernel.h", "step_kernel.h", "mimo_kernels.h",
                     "prefill_mimo_rows_kernel.h"],
    "step_mimo": ["scan_update.h", "step_kernel.h", "mimo_kernels.h"],
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
    oracle on inp["A"]; with `lam`, the exponential-trapezoidal oracle)."""
    import numpy as np

    import oracle

    threads = min(16, os.cpu_count() or 1)
    x = inp["x"][:, :, :channels]
    dl = inp["delta"][:, :, :channels]
    A = inp["A"][:channels] if scalar_a is None else scalar_a[:channels]
    args = [np.ascontiguousarray(t.float().numpy(), dtype=np.float64) for t in (x, dl, A, inp["B"], inp["C"])]
    fn = oracle.prefill_complex if complex_a else oracle.prefill if scalar_a is None else oracle.prefill_scalar_a
    t0 = time.perf_counter()
    form = "complex" if complex_a else "diagonal" if scalar_a is None else "scalar"
    if mimo and lam is not None:
        lm = np.ascontiguousarray(lam[:, :, :channels].float().numpy(), dtype=np.float64)
        oracle.prefill_mimo_trapezoid(args[0], args[1], lm, *args[2:], form=form, nthreads=threads)
    elif mimo:
        oracle.prefill_mimo(*args, form=form, nthreads=threads)
    elif lam is not None:
        lm = np.ascontiguousarray(lam[:, :, :channels].float().numpy(), dtype=np.float64)
        oracle.prefill_trapezoid(args[0], args[1], lm, *args[2:], form=form, nthreads=threads)
    else:
        fn(*args, nthreads=threads)
    dt = time.perf_counter() - t0
    elems = wl.batch * wl.L * channels
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next(line.split(":", 1)[1].strip() for line in fh if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": elems / dt, "unit": "elems/s", "cores": threads, "kind": "oracle",
            "sample": f"{wl.name}: batch {wl.batch}, all {wl.L} tokens, first {channels} of {wl.D} channels, "
                      f"N {wl.N}, fp64 ({dt:.1f} s on {cpu})"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
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
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the scan, time a plain device-to-device copy of MIB mebibytes (the reference "
                         "kernel for scaling the profiler's FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

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
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup):
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

    for _ in range(args.warmup):
        one_step()
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
    if wl.layers > 1:
        roofline = {"bound": "hbm", "achieved": round(alg_bytes / launches / (per_launch_ms * 1e-3) / 1e9, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
        roofline["frac"] = round(roofline["achieved"] / HBM_PEAK_GBPS, 4)
    else:
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
        roofline = {"bound": "alu", "achieved": round(achieved_tf, 2), "peak": round(peak_tf, 2), "unit": "TFLOP/s",
                    "frac": round(achieved_tf / peak_tf, 4)}
    roofline["traffic"] = None if (args.chunked or args.producer) else read_traffic(
        wl.name + ("_scalar_a" if args.scalar_a else "_complex_a" if args.complex_a else "")
        + ("_trapezoid" if args.trapezoid else "") + (f"_mimo{args.mimo}" if args.mimo else ""), launches)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "elems/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
    }
    if producer_info is not None:
        out["producer"] = producer_info
    if host_inp is not None and args.cpu_channels > 0 and wl.layers == 1:
        out["cpu_baseline"] = cpu_baseline(wl, host_inp, min(args.cpu_channels, wl.D),
                                           host_a if args.scalar_a else None, complex_a=args.complex_a,
                                           lam=host_inp.get("lam") if args.trapezoid else None, mimo=args.mimo)
        log(f"oracle sample: {out['cpu_baseline']['sample']}")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()

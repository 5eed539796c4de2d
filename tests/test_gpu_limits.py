"""The kernels at the C ABI's size limits: D = 2^24 channels and batch = 2^20 rows.

The large inputs are a small seeded case tiled along channels (or batch rows), so every channel
(row) of the large run must reproduce the small run's bits, and the small run is checked against
the oracle.  That a channel's output depends on nothing but its own inputs is the S6 recurrence
with a diagonal A (notes page "Jamba: A Hybrid Transformer-Mamba Language Model", section
"Mamba layer"): channel d's state and output depend only on its x, delta and row of A and on the
shared B and C, and the kernels compute each channel by the same instructions wherever it sits
(its position inside its 32-channel block is the same in both runs, as 256 is a multiple of 32).
The comparison runs on the GPU, on the raw bits."""
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, f64, say, to_dev

pytestmark = pytest.mark.gpu

MAX_D = 1 << 24
MAX_BATCH = 1 << 20


def raw(t):
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)


def tiled_equal(big, small, dim):
    """big is small repeated along dim: compare every copy, bit for bit, on the device."""
    reps = big.shape[dim] // small.shape[dim]
    shape = list(small.shape)
    shape[dim:dim + 1] = [reps, small.shape[dim]]
    return torch.equal(raw(big).reshape(shape), raw(small).unsqueeze(dim).expand(shape))


def test_prefill_at_the_channel_limit():
    inp = workloads.small_prefill(1, 70, 256, "bf16", seed=31)   # two tiles, the second ragged
    d = to_dev(inp)
    y_s, h_s = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_ref, h_ref = oracle.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    assert_parity(f64(y_s), y_ref, torch.bfloat16, "1x70x256 y")
    assert_parity(f64(h_s), h_ref, torch.bfloat16, "1x70x256 h_final")
    reps = MAX_D // 256
    say(f"prefill 1x70x{MAX_D} bf16: 256 channels tiled {reps} times")
    x, dl = d["x"].repeat(1, 1, reps), d["delta"].repeat(1, 1, reps)
    A = d["A"].repeat(reps, 1)
    y_b, h_b = jscan.prefill(x, dl, A, d["B"], d["C"])
    torch.cuda.synchronize()
    assert y_b.shape == (1, 70, MAX_D) and h_b.shape == (1, MAX_D, 16)
    assert tiled_equal(y_b, y_s, 2), "y of some channel differs from its copy in the small run"
    assert tiled_equal(h_b, h_s, 1), "h_final of some channel differs from its copy in the small run"


def test_step_at_the_channel_limit():
    wl = workloads.Workload("decode_limit", 83, 2, 1, 256, 16, "bf16", True, layers=1)
    inp = workloads.decode_layer_inputs(wl, 0)
    d = to_dev(inp)
    h_s = d["h0"].clone()
    y_s = jscan.step(h_s, d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_ref, h_ref = oracle.step(inp["h0"], inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    assert_parity(f64(y_s), y_ref, torch.bfloat16, "step 2x256 y")
    assert_parity(f64(h_s), h_ref, torch.bfloat16, "step 2x256 h")
    reps = MAX_D // 256
    say(f"step 2x{MAX_D} bf16: 256 channels tiled {reps} times")
    h_b = d["h0"].repeat(1, reps, 1)
    y_b = jscan.step(h_b, d["x"].repeat(1, reps), d["delta"].repeat(1, reps), d["A"].repeat(reps, 1), d["B"],
                     d["C"])
    torch.cuda.synchronize()
    assert tiled_equal(y_b, y_s, 1) and tiled_equal(h_b, h_s, 1)


def test_prefill_and_step_at_the_batch_limit():
    """2^20 sequences of 32 channels (one work-group each in the prefill), and a decode step over
    2^20 rows: each row reproduces its copy in a 16-row run."""
    inp = workloads.small_prefill(16, 3, 32, "bf16", seed=37)
    d = to_dev(inp)
    y_s, h_s = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_ref, h_ref = oracle.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    assert_parity(f64(y_s), y_ref, torch.bfloat16, "16x3x32 y")
    reps = MAX_BATCH // 16
    say(f"prefill {MAX_BATCH}x3x32 and step {MAX_BATCH}x32 bf16: 16 rows tiled {reps} times")
    big = {k: d[k].repeat(reps, 1, 1) for k in ("x", "delta", "B", "C")}
    y_b, h_b = jscan.prefill(big["x"], big["delta"], d["A"], big["B"], big["C"])
    torch.cuda.synchronize()
    assert tiled_equal(y_b, y_s, 0) and tiled_equal(h_b, h_s, 0)
    # one more token through the decode step, from the final states, every row strided
    hs, hb = h_s.clone(), h_b
    ys = jscan.step(hs, d["x"][:, 1], d["delta"][:, 1], d["A"], d["B"][:, 1], d["C"][:, 1])
    yb = jscan.step(hb, big["x"][:, 1], big["delta"][:, 1], d["A"], big["B"][:, 1], big["C"][:, 1])
    torch.cuda.synchronize()
    assert yb.shape == (MAX_BATCH, 32)
    assert tiled_equal(yb, ys, 0) and tiled_equal(hb, hs, 0)


def test_mimo_at_the_channel_limit():
    """The rank-8 MIMO prefill and step at D = 2^24 (rows of D * R = 2^27 values)."""
    R = 8
    wl = workloads.Workload("adhoc_mimo_limit", 611, 1, 66, 256, 16, "bf16", True)
    inp = workloads.mimo_inputs(wl, R, seed=3, threads=1)
    d = to_dev(inp)
    y_s, h_s = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_ref, h_ref = oracle.prefill_mimo(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    assert_parity(f64(y_s), y_ref, torch.bfloat16, "mimo 1x66x256 R8 y")
    reps = MAX_D // 256
    say(f"prefill_mimo 1x66x{MAX_D} R{R} bf16: 256 channels tiled {reps} times")
    x, dl, A = d["x"].repeat(1, 1, reps, 1), d["delta"].repeat(1, 1, reps), d["A"].repeat(reps, 1)
    y_b, h_b = jscan.prefill_mimo(x, dl, A, d["B"], d["C"])
    torch.cuda.synchronize()
    assert tiled_equal(y_b, y_s, 2) and tiled_equal(h_b, h_s, 1)
    del y_b
    # one more token through the MIMO step from the final states, token views of the same inputs
    hs, hb = h_s.clone(), h_b
    ys = jscan.step_mimo(hs, d["x"][:, 1], d["delta"][:, 1], d["A"], d["B"][:, 1], d["C"][:, 1])
    say(f"step_mimo 1x{MAX_D} R{R} bf16")
    yb = jscan.step_mimo(hb, x[:, 1], dl[:, 1], A, d["B"][:, 1], d["C"][:, 1])
    torch.cuda.synchronize()
    assert tiled_equal(yb, ys, 1) and tiled_equal(hb, hs, 1)

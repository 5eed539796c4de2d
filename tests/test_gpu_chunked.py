"""jscan_prefill_chunked (the time-parallel prefill) on the GPU against the fp64 oracle.

The segment composition rounds differently from the token-by-token walk, so the results
are checked to the tolerance (max|y - y_ref| <= tol * max|y_ref|, tol 1e-4 for fp32 inputs
and 2e-2 for bf16), not bit for bit.  What does hold exactly is checked exactly: the first
segment starts from the caller's state and is the sequential scan itself, a single segment
is jscan_prefill_resume, and repeated runs agree bit for bit."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_bf16_sums_close, assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu


def h0_for(batch, D, seed):
    g = np.random.default_rng([seed, 77])
    return torch.from_numpy(g.normal(0.0, 0.1, size=(batch, D, 16)).astype(np.float32))


@pytest.mark.parametrize("batch,L,D,dtype,chunk", [
    (1, 1000, 64, "f32", 0),       # automatic plan: 3 segments of 384 tokens, ragged last one
    (1, 1000, 64, "bf16", 64),     # 64-token segments
    (2, 777, 40, "f32", 100),      # D not a multiple of 32 (state-order sums), ragged segments
    (2, 777, 40, "bf16", 0),
    (3, 513, 96, "f32", 7),        # segments shorter than the kernel's 16-token main loop
    (1, 300, 32, "f32", 1),        # one token per segment; the carry's groups hold 19 segments
    (1, 4096, 1024, "bf16", 0),    # automatic plan: 16 segments of 256 tokens
    (2, 3000, 1000, "bf16", 0),    # 10 segments of 320 tokens a sequence; a partly filled work-group
])
@pytest.mark.parametrize("with_h0", [False, True])
def test_chunked_matches_oracle(batch, L, D, dtype, chunk, with_h0):
    inp = workloads.small_prefill(batch, L, D, dtype, seed=3)
    h0 = h0_for(batch, D, 5) if with_h0 else None
    dev = to_dev(inp)
    what = f"chunked {batch}x{L}x{D} {dtype} chunk={chunk} h0={with_h0}"
    say(what, "workspace", jscan.chunked_workspace_bytes(batch, L, D, chunk), "bytes")
    y, h = jscan.prefill_chunked(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"],
                                 h0=None if h0 is None else h0.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0)
    td = dev["x"].dtype
    assert_parity(f64(y), y_ref, td, f"{what} y")
    assert_parity(f64(h), h_ref, td, f"{what} h_final")


@pytest.mark.parametrize("batch,L,D,dtype,chunk", [(1, 1000, 64, "bf16", 192), (2, 777, 40, "f32", 100)])
def test_first_segment_is_the_sequential_scan(batch, L, D, dtype, chunk):
    """Segment 0 starts from h0 itself, so its states are the sequential prefill's.  With fp32
    output its y is bit-identical too (the same sums in the same order); with bf16 output the
    sequential prefill sums over states on the matrix cores from bf16-rounded partials, so y
    agrees to that rounding."""
    inp = to_dev(workloads.small_prefill(batch, L, D, dtype, seed=4))
    h0 = h0_for(batch, D, 6).cuda()
    y_seq, _ = jscan.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0)
    y_chk, _ = jscan.prefill_chunked(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0, chunk=chunk)
    torch.cuda.synchronize()
    a, b = y_chk[:, :chunk], y_seq[:, :chunk]
    if dtype == "f32":
        assert torch.equal(bits(a), bits(b))
    else:
        assert_bf16_sums_close(a, b, "first segment y")


@pytest.mark.parametrize("chunk", [0, 4096, 100000])
def test_single_segment_is_prefill_resume(chunk):
    """A chunk covering the sequence (or automatic chunking of a shape that already fills
    the GPU) is exactly jscan_prefill_resume; no workspace is needed."""
    batch, L, D = (1, 4096, 8192) if chunk == 0 else (1, 4096, 256)
    inp = to_dev(workloads.small_prefill(batch, L, D, "bf16", seed=8))
    assert jscan.chunked_workspace_bytes(batch, L, D, chunk) == 0
    y0, h0 = jscan.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    y1, h1 = jscan.prefill_chunked(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(bits(y0), bits(y1)) and torch.equal(bits(h0), bits(h1))


def test_chunked_is_deterministic_and_in_place():
    inp = to_dev(workloads.small_prefill(1, 2000, 512, "bf16", seed=9))
    h0 = h0_for(1, 512, 10).cuda()
    ya, ha = jscan.prefill_chunked(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0, chunk=256)
    yb, hb = jscan.prefill_chunked(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0, chunk=256)
    hc = h0.clone()   # h0 == h_final: the state updated in place
    yc, _ = jscan.prefill_chunked(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=hc, h_final=hc, chunk=256)
    torch.cuda.synchronize()
    assert torch.equal(bits(ya), bits(yb)) and torch.equal(bits(ha), bits(hb))
    assert torch.equal(bits(ya), bits(yc)) and torch.equal(bits(ha), bits(hc))


def test_chunked_agrees_with_sequential_gpu_scan_on_zero_A():
    """A = 0 makes every decay exactly 1, so the composition is plain addition of integers
    (delta = 0.5, x = 1, B = 2, C = 1 give h_t = t + 1 exactly): the chunked y and state
    must equal the sequential ones bit for bit."""
    L, D = 3000, 64
    x = torch.ones(1, L, D, dtype=torch.bfloat16, device="cuda")
    dl = torch.full_like(x, 0.5)
    B = torch.full((1, L, 16), 2.0, dtype=torch.bfloat16, device="cuda")
    C = torch.ones_like(B)
    A = torch.zeros(D, 16, device="cuda")
    y0, h0 = jscan.prefill(x, dl, A, B, C)
    y1, h1 = jscan.prefill_chunked(x, dl, A, B, C, chunk=128)
    torch.cuda.synchronize()
    assert torch.equal(bits(y0), bits(y1)) and torch.equal(bits(h0), bits(h1))
    assert float(h1[0, 0, 0]) == L


@pytest.mark.timeout(600)
def test_prefill_64k_tp8_chunked_every_channel():
    """The channel-sharded 64K prompt (D = 1024 per GPU) through the automatic time-parallel
    path, in the launch configuration the benchmark times, against the oracle on every
    channel over all 65536 tokens."""
    wl = workloads.get("prefill_64k_tp8")
    say("generating prefill_64k_tp8 inputs")
    inp = workloads.prefill_inputs(wl)
    d = to_dev(inp)
    y, h = jscan.prefill_chunked(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_seq, h_seq = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    say(f"oracle on all {wl.D} channels x {wl.L} tokens")
    y_ref, h_ref = oracle.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], nthreads=16)
    assert_parity(f64(y), y_ref, torch.bfloat16, "prefill_64k_tp8 chunked y")
    assert_parity(f64(h), h_ref, torch.bfloat16, "prefill_64k_tp8 chunked h_final")
    assert_parity(f64(y_seq), y_ref, torch.bfloat16, "prefill_64k_tp8 sequential y")
    assert_parity(f64(h_seq), h_ref, torch.bfloat16, "prefill_64k_tp8 sequential h_final")

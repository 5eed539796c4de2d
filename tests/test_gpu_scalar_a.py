"""Scaled-identity A (A[d, n] = a[d], the Mamba-2 form): jscan_prefill_scalar_a and
jscan_step_scalar_a on the GPU.

These kernels evaluate the channel's decay once per (token, channel) by the same fp32
expression the general kernels evaluate once per state element, so on the expanded
A[d, n] = a[d] every output must equal the general path's bit for bit; that is checked on
both prefill kernels (row-mapped and lane), ragged shapes, a resumed state, the decode step
and the full 64K workload.  Against the fp64 oracle (oracle.prefill_scalar_a) the outputs
meet the usual tolerance, max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2 bf16)."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu


def scalar_case(batch, L, D, dtype, seed=0):
    inp = workloads.small_prefill(batch, L, D, dtype, seed=seed)
    wl = workloads.Workload(f"adhoc_a_{batch}x{L}x{D}", 300 + D % 97, batch, L, D, 16, dtype, True)
    inp["a"] = workloads.draw_scalar_a(wl, seed=seed)
    return inp


def expanded(a):
    return a[:, None].expand(-1, 16).contiguous()


@pytest.mark.parametrize("batch,L,D,dtype,with_h0", [
    (1, 1000, 512, "bf16", False),   # row-mapped kernel, ragged last tile
    (2, 300, 1024, "f32", True),     # row-mapped fp32, batch 2, resumed
    (1, 63, 128, "bf16", True),      # shorter than one tile
    (1, 1, 64, "bf16", False),       # one token
    (2, 777, 40, "f32", False),      # D not a multiple of 32: lane kernel
    (9, 70, 8192, "bf16", True),     # batch * D above 65536 (row-mapped kernel, many rows)
    (3, 100, 200, "bf16", True),     # D not a multiple of 32 (lane kernel), bf16
])
def test_bit_identical_to_general_path(batch, L, D, dtype, with_h0):
    inp = to_dev(scalar_case(batch, L, D, dtype, seed=L))
    h0 = (torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(2)) * 0.3).cuda() if with_h0 else None
    say(f"scalar-a {batch}x{L}x{D} {dtype} h0={with_h0}")
    y1, h1 = jscan.prefill_scalar_a(inp["x"], inp["delta"], inp["a"], inp["B"], inp["C"], h0=h0)
    y2, h2 = jscan.prefill(inp["x"], inp["delta"], expanded(inp["a"]), inp["B"], inp["C"], h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y2)), "y differs from the general path"
    assert torch.equal(bits(h1), bits(h2)), "h_final differs from the general path"


@pytest.mark.parametrize("batch,L,D,dtype", [(1, 4096, 8192, "bf16"), (2, 777, 40, "f32"), (1, 1000, 256, "f32")])
def test_matches_oracle(batch, L, D, dtype):
    host = scalar_case(batch, L, D, dtype, seed=7)
    inp = to_dev(host)
    y, h = jscan.prefill_scalar_a(inp["x"], inp["delta"], inp["a"], inp["B"], inp["C"])
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_scalar_a(host["x"], host["delta"], host["a"], host["B"], host["C"])
    td = inp["x"].dtype
    assert_parity(f64(y), y_ref, td, f"scalar-a {batch}x{L}x{D} {dtype} y")
    assert_parity(f64(h), h_ref, td, f"scalar-a {batch}x{L}x{D} {dtype} h_final")


def test_resume_splits_exactly():
    """Scanning [0, L1) then resuming over [L1, L) equals one scan of [0, L), bit for bit."""
    inp = to_dev(scalar_case(1, 1000, 512, "bf16", seed=3))
    y, h = jscan.prefill_scalar_a(inp["x"], inp["delta"], inp["a"], inp["B"], inp["C"])
    L1 = 448
    part = {k: (v[:, :L1].contiguous(), v[:, L1:].contiguous()) for k, v in inp.items() if k != "a"}
    ya, ha = jscan.prefill_scalar_a(part["x"][0], part["delta"][0], inp["a"], part["B"][0], part["C"][0])
    yb, hb = jscan.prefill_scalar_a(part["x"][1], part["delta"][1], inp["a"], part["B"][1], part["C"][1], h0=ha)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.cat([ya, yb], 1)), bits(y)) and torch.equal(bits(hb), bits(h))


@pytest.mark.parametrize("batch,D,dtype", [(256, 8192, "bf16"), (3, 40, "f32")])
def test_step_bit_identical_to_general_step(batch, D, dtype):
    g = torch.Generator().manual_seed(batch + D)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    h = (torch.randn(batch, D, 16, generator=g) * 0.1).cuda()
    x, dl = torch.randn(batch, D, generator=g).to(td).cuda(), (torch.rand(batch, D, generator=g) * 0.5).to(td).cuda()
    B, C = torch.randn(batch, 16, generator=g).to(td).cuda(), torch.randn(batch, 16, generator=g).to(td).cuda()
    wl = workloads.Workload("adhoc_step", 311, batch, 1, D, 16, dtype, True)
    a = workloads.draw_scalar_a(wl).cuda()
    h1, h2 = h.clone(), h.clone()
    y1 = jscan.step_scalar_a(h1, x, dl, a, B, C)
    y2 = jscan.step(h2, x, dl, expanded(a), B, C)
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y2)) and torch.equal(bits(h1), bits(h2))
    y_ref, h_ref = oracle.step_scalar_a(h.cpu(), x.cpu(), dl.cpu(), a.cpu(), B.cpu(), C.cpu())
    assert_parity(f64(y1), y_ref, td, f"scalar-a step {batch}x{D} y")
    assert_parity(f64(h1), h_ref, td, f"scalar-a step {batch}x{D} h")


def test_prefill_state_equals_step_chain():
    """h_final of the scaled-identity prefill equals L scaled-identity decode steps bit for bit."""
    inp = to_dev(scalar_case(2, 200, 256, "bf16", seed=5))
    h0 = (torch.randn(2, 256, 16, generator=torch.Generator().manual_seed(9)) * 0.2).cuda()
    y, h = jscan.prefill_scalar_a(inp["x"], inp["delta"], inp["a"], inp["B"], inp["C"], h0=h0)
    hs = h0.clone()
    for t in range(200):
        jscan.step_scalar_a(hs, inp["x"][:, t], inp["delta"][:, t], inp["a"], inp["B"][:, t], inp["C"][:, t])
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h))


def test_prefill_64k_full_size():
    """The 64K x 8192 workload with a scaled-identity A, in the launch configuration the
    benchmark times: bit-identical to the general kernel on the expanded A over every output,
    and within tolerance of the oracle on sampled channels over all tokens."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k inputs")
    host = workloads.prefill_inputs(wl)
    a = workloads.draw_scalar_a(wl)
    d = to_dev(host)
    ad = a.cuda()
    y1, h1 = jscan.prefill_scalar_a(d["x"], d["delta"], ad, d["B"], d["C"])
    torch.cuda.synchronize()
    y2, h2 = jscan.prefill(d["x"], d["delta"], expanded(ad), d["B"], d["C"])
    torch.cuda.synchronize()
    same_y = torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    same_h = torch.equal(h1.view(torch.int32), h2.view(torch.int32))
    del y2
    assert same_y and same_h, "the 64K scaled-identity scan differs from the general path"
    chans = sorted(set([0, 1, 31, 32, 4095, 8191] + np.random.default_rng(4).choice(wl.D, 10, replace=False).tolist()))
    say(f"oracle on {len(chans)} channels x {wl.L} tokens")
    y_ref, h_ref = oracle.prefill_scalar_a(host["x"][:, :, chans], host["delta"][:, :, chans], a[chans], host["B"],
                                           host["C"])
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y1.index_select(2, idx)), y_ref, torch.bfloat16, "scalar-a 64K y (sampled)")
    assert_parity(f64(h1.index_select(1, idx)), h_ref, torch.bfloat16, "scalar-a 64K h_final (sampled)")

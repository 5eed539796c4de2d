"""Complex-valued state (the Mamba-3 form: states 2k, 2k+1 of a channel as one complex state,
A[d, 2k], A[d, 2k+1] the real and imaginary parts of its diagonal entry) on the GPU:
jscan_prefill_complex and jscan_step_complex against the fp64 oracle (oracle.prefill_complex),
max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2 bf16), on both prefill kernels.  Exact
properties are checked exactly: the prefill's final state equals the step chain bit for bit,
a resumed scan equals one long scan, and with every imaginary part zero the kernels compute
the real scan on A[d, 2k+1] = A[d, 2k] bit for bit (cos 0 = 1 and sin 0 = 0 exactly)."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu


def complex_case(batch, L, D, dtype, seed=0):
    inp = workloads.small_prefill(batch, L, D, dtype, seed=seed)
    wl = workloads.Workload(f"adhoc_c_{batch}x{L}x{D}", 400 + D % 97, batch, L, D, 16, dtype, True)
    inp["A"] = workloads.draw_complex_a(wl, seed=seed)
    return inp


def h0_for(batch, D, seed):
    return (torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(seed)) * 0.3)


@pytest.mark.parametrize("batch,L,D,dtype,with_h0", [
    (1, 1000, 512, "bf16", False),   # row-mapped kernel, ragged last tile
    (2, 300, 1024, "f32", True),     # row-mapped fp32, resumed
    (1, 63, 128, "bf16", True),      # shorter than one tile
    (1, 1, 64, "f32", False),        # one token
    (2, 777, 40, "f32", True),       # D not a multiple of 32: lane kernel
    (3, 100, 200, "bf16", False),    # lane kernel, bf16
])
def test_matches_oracle(batch, L, D, dtype, with_h0):
    host = complex_case(batch, L, D, dtype, seed=L + D)
    h0 = h0_for(batch, D, 3) if with_h0 else None
    d = to_dev(host)
    say(f"complex {batch}x{L}x{D} {dtype} h0={with_h0}")
    y, h = jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=None if h0 is None else h0.cuda())
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_complex(host["x"], host["delta"], host["A"], host["B"], host["C"], h0=h0)
    td = d["x"].dtype
    assert_parity(f64(y), y_ref, td, f"complex {batch}x{L}x{D} y")
    assert_parity(f64(h), h_ref, td, f"complex {batch}x{L}x{D} h_final")


def test_prefill_4k_matches_oracle():
    """The 4K-token Jamba-width shape (1 x 4096 x 8192, bf16) against the full oracle."""
    host = complex_case(1, 4096, 8192, "bf16", seed=9)
    d = to_dev(host)
    y, h = jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_complex(host["x"], host["delta"], host["A"], host["B"], host["C"])
    assert_parity(f64(y), y_ref, torch.bfloat16, "complex 4K y")
    assert_parity(f64(h), h_ref, torch.bfloat16, "complex 4K h_final")


@pytest.mark.parametrize("batch,L,D,dtype", [(1, 1000, 512, "bf16"), (2, 777, 40, "f32")])
def test_no_rotation_is_the_real_scan_bitwise(batch, L, D, dtype):
    d = to_dev(complex_case(batch, L, D, dtype, seed=5))
    A = d["A"].clone()
    A[:, 1::2] = 0.0
    Ar = A.clone()
    Ar[:, 1::2] = A[:, 0::2]
    y1, h1 = jscan.prefill_complex(d["x"], d["delta"], A, d["B"], d["C"])
    y2, h2 = jscan.prefill(d["x"], d["delta"], Ar, d["B"], d["C"])
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y2)) and torch.equal(bits(h1), bits(h2))


@pytest.mark.parametrize("batch,L,D", [(2, 200, 256), (3, 60, 40)])
def test_prefill_state_equals_step_chain(batch, L, D):
    d = to_dev(complex_case(batch, L, D, "bf16", seed=7))
    h0 = h0_for(batch, D, 4).cuda()
    y, h = jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0)
    hs = h0.clone()
    for t in range(L):
        jscan.step_complex(hs, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t])
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h))


def test_resume_splits_exactly():
    d = to_dev(complex_case(1, 1000, 512, "bf16", seed=8))
    y, h = jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"])
    L1 = 320
    part = {k: (v[:, :L1].contiguous(), v[:, L1:].contiguous()) for k, v in d.items() if k != "A"}
    ya, ha = jscan.prefill_complex(part["x"][0], part["delta"][0], d["A"], part["B"][0], part["C"][0])
    yb, hb = jscan.prefill_complex(part["x"][1], part["delta"][1], d["A"], part["B"][1], part["C"][1], h0=ha)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.cat([ya, yb], 1)), bits(y)) and torch.equal(bits(hb), bits(h))


@pytest.mark.parametrize("batch,D,dtype", [(256, 8192, "bf16"), (3, 40, "f32")])
def test_step_matches_oracle(batch, D, dtype):
    g = torch.Generator().manual_seed(batch + D)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.randn(batch, D, 16, generator=g) * 0.1
    x, dl = torch.randn(batch, D, generator=g).to(td), (torch.rand(batch, D, generator=g) * 0.5).to(td)
    B, C = torch.randn(batch, 16, generator=g).to(td), torch.randn(batch, 16, generator=g).to(td)
    A = workloads.draw_complex_a(workloads.Workload("adhoc_cs", 411, batch, 1, D, 16, dtype, True))
    hd = h.cuda()
    y = jscan.step_complex(hd, x.cuda(), dl.cuda(), A.cuda(), B.cuda(), C.cuda())
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.step_complex(h, x, dl, A, B, C)
    assert_parity(f64(y), y_ref, td, f"complex step {batch}x{D} y")
    assert_parity(f64(hd), h_ref, td, f"complex step {batch}x{D} h")


def test_prefill_64k_sampled_parity():
    """The 64K x 8192 workload with a complex A, in the launch configuration the benchmark
    times, against the oracle on sampled channels over all tokens."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k inputs")
    host = workloads.prefill_inputs(wl)
    host["A"] = workloads.draw_complex_a(wl)
    d = to_dev(host)
    y, h = jscan.prefill_complex(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    chans = sorted(set([0, 1, 31, 32, 4095, 8191] + np.random.default_rng(6).choice(wl.D, 10, replace=False).tolist()))
    say(f"oracle on {len(chans)} channels x {wl.L} tokens")
    y_ref, h_ref = oracle.prefill_complex(host["x"][:, :, chans], host["delta"][:, :, chans], host["A"][chans],
                                          host["B"], host["C"])
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, "complex 64K y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, "complex 64K h_final (sampled)")

"""The multi-input, multi-output scan (MIMO: R inputs and R outputs per channel, B_t and C_t
N x R) on the GPU, for each form of A: jscan_prefill_mimo and jscan_step_mimo against the fp64
oracle (oracle.prefill_mimo / step_mimo), max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2
bf16).  Exact properties are checked exactly: the prefill's final state equals the step chain
bit for bit, and with R = 1 the state is the single-input entry point's bit for bit (y agrees
to rounding: the kernels sum C h over the states in different orders)."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu

FORMS = ["diagonal", "scalar", "complex"]


def mimo_case(batch, L, D, R, dtype, form, seed=0):
    wl = workloads.Workload(f"adhoc_m_{batch}x{L}x{D}", 600 + (D + 7 * L) % 97, batch, L, D, 16, dtype, True)
    inp = workloads.mimo_inputs(wl, R, seed=seed, threads=1)
    if form == "scalar":
        inp["A"] = workloads.draw_scalar_a(wl, seed=seed)
    elif form == "complex":
        inp["A"] = workloads.draw_complex_a(wl, seed=seed)
    return inp


def h0_for(batch, D, seed):
    return torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(seed)) * 0.3


def siso(form):
    return {"diagonal": jscan.prefill, "scalar": jscan.prefill_scalar_a, "complex": jscan.prefill_complex}[form]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,R,dtype,with_h0", [
    (1, 300, 256, 4, "bf16", False),
    (2, 100, 40, 4, "f32", True),      # D not a multiple of 64: a partial wave
    (1, 200, 128, 1, "bf16", True),
    (2, 150, 64, 2, "f32", False),
    (1, 120, 64, 8, "bf16", True),
    (1, 1, 64, 4, "f32", False),       # one token
])
def test_matches_oracle(form, batch, L, D, R, dtype, with_h0):
    host = mimo_case(batch, L, D, R, dtype, form, seed=L + D + R)
    h0 = h0_for(batch, D, 3) if with_h0 else None
    d = to_dev(host)
    what = f"mimo {form} {batch}x{L}x{D} R={R} {dtype} h0={with_h0}"
    say(what)
    y, h = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=None if h0 is None else h0.cuda(),
                              form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_mimo(host["x"], host["delta"], host["A"], host["B"], host["C"], h0=h0, form=form)
    td = d["x"].dtype
    assert_parity(f64(y), y_ref, td, f"{what} y")
    assert_parity(f64(h), h_ref, td, f"{what} h_final")


@pytest.mark.parametrize("form", FORMS)
def test_prefill_4k_matches_oracle(form):
    """The 4K-token Jamba-width shape (1 x 4096 x 8192, rank 4, bf16) against the full oracle."""
    host = mimo_case(1, 4096, 8192, 4, "bf16", form, seed=9)
    d = to_dev(host)
    say(f"mimo {form} 4K")
    y, h = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_mimo(host["x"], host["delta"], host["A"], host["B"], host["C"], form=form)
    assert_parity(f64(y), y_ref, torch.bfloat16, f"mimo {form} 4K y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"mimo {form} 4K h_final")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,dtype", [(1, 500, 256, "bf16"), (2, 300, 40, "f32")])
def test_rank_one_is_the_single_input_scan(form, batch, L, D, dtype):
    d = to_dev(mimo_case(batch, L, D, 1, dtype, form, seed=5))
    h0 = h0_for(batch, D, 6).cuda()
    y1, h1 = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, form=form)
    y2, h2 = siso(form)(d["x"][..., 0].contiguous(), d["delta"], d["A"], d["B"][..., 0].contiguous(),
                        d["C"][..., 0].contiguous(), h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(bits(h1), bits(h2)), "rank-one state differs from the single-input scan's"
    assert_parity(f64(y1[..., 0]), f64(y2), d["x"].dtype, f"mimo {form} rank one y vs single input")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,R", [(2, 100, 256, 4), (3, 40, 40, 2), (1, 60, 64, 8)])
def test_prefill_state_equals_step_chain(form, batch, L, D, R):
    d = to_dev(mimo_case(batch, L, D, R, "bf16", form, seed=7))
    h0 = h0_for(batch, D, 4).cuda()
    y, h = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, form=form)
    hs = h0.clone()
    ys = [jscan.step_mimo(hs, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t], form=form).clone()
          for t in range(L)]
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h)), "step chain state differs from the prefill's"
    assert_parity(f64(torch.stack(ys, 1)), f64(y), torch.bfloat16, f"mimo {form} step chain y")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,D,R,dtype", [(256, 8192, 4, "bf16"), (3, 40, 2, "f32"), (5, 64, 8, "bf16")])
def test_step_matches_oracle(form, batch, D, R, dtype):
    wl = workloads.Workload("adhoc_ms", 611, batch, 1, D, 16, dtype, True)
    g = torch.Generator().manual_seed(batch + D + R)
    td = wl.torch_dtype
    h = torch.randn(batch, D, 16, generator=g) * 0.1
    x = torch.randn(batch, D, R, generator=g).to(td)
    dl = (torch.rand(batch, D, generator=g) * 0.5).to(td)
    B, C = (torch.randn(batch, 16, R, generator=g).to(td) for _ in range(2))
    A = {"diagonal": workloads.draw_A, "scalar": workloads.draw_scalar_a, "complex": workloads.draw_complex_a}[form](wl)
    hd = h.cuda()
    y = jscan.step_mimo(hd, x.cuda(), dl.cuda(), A.cuda(), B.cuda(), C.cuda(), form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.step_mimo(h, x, dl, A, B, C, form=form)
    assert_parity(f64(y), y_ref, td, f"mimo {form} step {batch}x{D} R={R} y")
    assert_parity(f64(hd), h_ref, td, f"mimo {form} step {batch}x{D} R={R} h")


def test_decode_layer_matches_oracle():
    """One layer of the 256-sequence decode workload at rank 4, in the launch configuration the
    benchmark times."""
    host = workloads.decode_layer_mimo_inputs("decode_256x28", 3, 4)
    d = to_dev(host)
    y = jscan.step_mimo(d["h0"], d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.step_mimo(host["h0"], host["x"], host["delta"], host["A"], host["B"], host["C"])
    assert_parity(f64(y), y_ref, torch.bfloat16, "mimo decode layer y")
    assert_parity(f64(d["h0"]), h_ref, torch.bfloat16, "mimo decode layer h")


@pytest.mark.parametrize("name", ["prefill_16x4k", "prefill_64k"])
def test_bench_workloads_sampled_parity(name):
    """The benchmark's MIMO workloads (rank 4) against the oracle on sampled channels over all tokens."""
    wl = workloads.get(name)
    say(f"generating {name} rank-4 inputs")
    host = workloads.mimo_inputs(wl, 4)
    d = to_dev(host)
    y, h = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    del d
    chans = sorted(set([0, 63, 64, wl.D - 1] + np.random.default_rng(2).choice(wl.D, 6, replace=False).tolist()))
    say(f"oracle on {len(chans)} channels")
    y_ref, h_ref = oracle.prefill_mimo(host["x"][:, :, chans], host["delta"][:, :, chans], host["A"][chans],
                                       host["B"], host["C"])
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, f"mimo {name} y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, f"mimo {name} h_final (sampled)")

"""The MIMO scan with the exponential-trapezoidal rule (both Mamba-3 changes together) on the GPU,
for each form of A: jscan_prefill_mimo_trapezoid and jscan_step_mimo_trapezoid against the fp64
oracle (oracle.prefill_mimo_trapezoid), max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32, 2e-2
bf16).  Exact properties are checked exactly: with lam = 1 the state is the MIMO entry point's
bit for bit, the prefill's final state equals the step chain's, and a scan resumed from
(h, previous token) equals the whole scan."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu

FORMS = ["diagonal", "scalar", "complex"]


def case(batch, L, D, R, dtype, form, seed=0):
    wl = workloads.Workload(f"adhoc_mt_{batch}x{L}x{D}", 700 + (D + 5 * L) % 89, batch, L, D, 16, dtype, True)
    inp = workloads.mimo_inputs(wl, R, seed=seed, threads=1)
    inp["lam"] = workloads.lam_inputs(wl, seed=seed, threads=1)
    if form == "scalar":
        inp["A"] = workloads.draw_scalar_a(wl, seed=seed)
    elif form == "complex":
        inp["A"] = workloads.draw_complex_a(wl, seed=seed)
    return inp


def prev_token(batch, D, R, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.randn(batch, D, R, generator=g).to(td), torch.randn(batch, 16, R, generator=g).to(td)


def h0_for(batch, D, seed):
    return torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(seed)) * 0.3


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,R,dtype,with_prev", [
    (1, 300, 256, 4, "bf16", False),   # row-mapped kernel, 16-token tiles, ragged
    (2, 100, 64, 2, "f32", True),      # row-mapped kernel, rank 2
    (1, 120, 64, 8, "bf16", True),     # rank 8: lane kernel
    (2, 77, 40, 4, "f32", True),       # D not a multiple of 32: lane kernel
    (1, 1, 64, 4, "f32", True),        # one token
    (1, 200, 128, 1, "bf16", True),    # rank 1: the single-input trapezoidal kernels
])
def test_matches_oracle(form, batch, L, D, R, dtype, with_prev):
    host = case(batch, L, D, R, dtype, form, seed=L + D + R)
    h0 = h0_for(batch, D, 3) if with_prev else None
    xp, bp = prev_token(batch, D, R, dtype, 4) if with_prev else (None, None)
    d = to_dev(host)
    what = f"mimo trapezoid {form} {batch}x{L}x{D} R={R} {dtype} prev={with_prev}"
    say(what)
    y, h = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"],
                                        h0=None if h0 is None else h0.cuda(),
                                        x_prev=None if xp is None else xp.cuda(),
                                        B_prev=None if bp is None else bp.cuda(), form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_mimo_trapezoid(host["x"], host["delta"], host["lam"], host["A"], host["B"], host["C"],
                                                 h0=h0, x_prev=xp, B_prev=bp, form=form)
    td = d["x"].dtype
    assert_parity(f64(y), y_ref, td, f"{what} y")
    assert_parity(f64(h), h_ref, td, f"{what} h_final")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,R,dtype", [(1, 300, 256, 4, "bf16"), (2, 100, 64, 2, "f32"), (1, 60, 64, 8, "bf16")])
def test_lambda_one_is_mimo_bitwise(form, batch, L, D, R, dtype):
    d = to_dev(case(batch, L, D, R, dtype, form, seed=5))
    h0 = h0_for(batch, D, 6).cuda()
    xp, bp = (v.cuda() for v in prev_token(batch, D, R, dtype, 7))
    y1, h1 = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], torch.ones_like(d["delta"]), d["A"], d["B"], d["C"],
                                          h0=h0, x_prev=xp, B_prev=bp, form=form)
    y2, h2 = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, form=form)
    torch.cuda.synchronize()
    assert torch.equal(bits(h1), bits(h2)), "lam = 1 state differs from the MIMO scan's"
    assert_parity(f64(y1), f64(y2), d["x"].dtype, f"mimo trapezoid {form} lam = 1 y")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,R,with_prev", [(2, 100, 256, 4, True), (1, 70, 64, 2, False), (3, 40, 40, 4, True),
                                                   (1, 50, 64, 8, True)])
def test_prefill_state_equals_step_chain(form, batch, L, D, R, with_prev):
    d = to_dev(case(batch, L, D, R, "bf16", form, seed=7))
    h0 = h0_for(batch, D, 4).cuda()
    if with_prev:
        xp, bp = (v.cuda() for v in prev_token(batch, D, R, "bf16", 8))
    else:
        xp, bp = torch.zeros_like(d["x"][:, 0]), torch.zeros_like(d["B"][:, 0])
    y, h = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], h0=h0,
                                        x_prev=xp if with_prev else None, B_prev=bp if with_prev else None, form=form)
    # token rows with the previous token in front, so that every row the step reads shares one stride
    pad = lambda first, v: torch.cat([first[:, None], v], 1)  # noqa: E731
    X, Bx = pad(xp, d["x"]), pad(bp, d["B"])
    Dl, Lm = (pad(torch.zeros_like(d[k][:, 0]), d[k]) for k in ("delta", "lam"))
    Cx = pad(torch.zeros_like(d["C"][:, 0]), d["C"])
    hs = h0.clone()
    ys = [jscan.step_mimo_trapezoid(hs, X[:, t], Bx[:, t], X[:, t + 1], Dl[:, t + 1], Lm[:, t + 1], d["A"],
                                    Bx[:, t + 1], Cx[:, t + 1], form=form).clone() for t in range(L)]
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h)), "step chain state differs from the prefill's"
    assert_parity(f64(torch.stack(ys, 1)), f64(y), torch.bfloat16, f"mimo trapezoid {form} step chain y")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("R", [2, 4])
def test_resume_splits_exactly(form, R):
    d = to_dev(case(1, 500, 256, R, "bf16", form, seed=8))
    y, h = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
    L1 = 176
    part = {k: (v[:, :L1].contiguous(), v[:, L1:].contiguous()) for k, v in d.items() if k != "A"}
    ya, ha = jscan.prefill_mimo_trapezoid(part["x"][0], part["delta"][0], part["lam"][0], d["A"], part["B"][0],
                                          part["C"][0], form=form)
    yb, hb = jscan.prefill_mimo_trapezoid(part["x"][1], part["delta"][1], part["lam"][1], d["A"], part["B"][1],
                                          part["C"][1], h0=ha, x_prev=d["x"][:, L1 - 1].contiguous(),
                                          B_prev=d["B"][:, L1 - 1].contiguous(), form=form)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.cat([ya, yb], 1)), bits(y)) and torch.equal(bits(hb), bits(h))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,D,R,dtype", [(256, 8192, 4, "bf16"), (3, 40, 2, "f32")])
def test_step_matches_oracle(form, batch, D, R, dtype):
    wl = workloads.Workload("adhoc_mts", 711, batch, 1, D, 16, dtype, True)
    g = torch.Generator().manual_seed(batch + D + R)
    td = wl.torch_dtype
    h = torch.randn(batch, D, 16, generator=g) * 0.1
    x, xp = (torch.randn(batch, D, R, generator=g).to(td) for _ in range(2))
    dl = (torch.rand(batch, D, generator=g) * 0.5).to(td)
    lam = torch.rand(batch, D, generator=g).to(td)
    B, C, Bp = (torch.randn(batch, 16, R, generator=g).to(td) for _ in range(3))
    A = {"diagonal": workloads.draw_A, "scalar": workloads.draw_scalar_a, "complex": workloads.draw_complex_a}[form](wl)
    hd = h.cuda()
    y = jscan.step_mimo_trapezoid(hd, xp.cuda(), Bp.cuda(), x.cuda(), dl.cuda(), lam.cuda(), A.cuda(), B.cuda(),
                                  C.cuda(), form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.step_mimo_trapezoid(h, xp, Bp, x, dl, lam, A, B, C, form=form)
    assert_parity(f64(y), y_ref, td, f"mimo trapezoid {form} step {batch}x{D} R={R} y")
    assert_parity(f64(hd), h_ref, td, f"mimo trapezoid {form} step {batch}x{D} R={R} h")


def test_prefill_64k_sampled_parity():
    """The 64K x 8192 workload at rank 4 with the trapezoidal rule, in the launch configuration the
    benchmark times, against the oracle on sampled channels over all tokens."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k rank-4 inputs with lam")
    host = workloads.mimo_inputs(wl, 4)
    host["lam"] = workloads.lam_inputs(wl)
    d = to_dev(host)
    y, h = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    del d
    chans = sorted(set([0, 31, 32, 8191] + np.random.default_rng(4).choice(wl.D, 6, replace=False).tolist()))
    say(f"oracle on {len(chans)} channels")
    y_ref, h_ref = oracle.prefill_mimo_trapezoid(host["x"][:, :, chans], host["delta"][:, :, chans],
                                                 host["lam"][:, :, chans], host["A"][chans], host["B"], host["C"])
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, "mimo trapezoid 64K y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, "mimo trapezoid 64K h_final (sampled)")

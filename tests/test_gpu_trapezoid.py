"""The exponential-trapezoidal rule (the Mamba-3 discretisation) on the GPU, for each form of A:
jscan_prefill_trapezoid and jscan_step_trapezoid against the fp64 oracle
(oracle.prefill_trapezoid / step_trapezoid), max|y - y_ref| <= tol * max|y_ref| (1e-4 fp32,
2e-2 bf16), on both prefill kernels.  Exact properties are checked exactly: the prefill's
final state equals the step chain bit for bit, a scan resumed from (h, previous token) equals
the whole scan, and with lam = 1 every kernel computes the Euler rule of the other entry
points bit for bit.  (The step chain's y equals the prefill's only to rounding: the kernels
sum C h over the 16 states in different orders.)"""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu

FORMS = ["diagonal", "scalar", "complex"]


def trap_case(batch, L, D, dtype, form, seed=0):
    inp = workloads.small_prefill(batch, L, D, dtype, seed=seed)
    wl = workloads.Workload(f"adhoc_t_{batch}x{L}x{D}", 500 + D % 89, batch, L, D, 16, dtype, True)
    inp["lam"] = workloads.lam_inputs(wl, seed=seed, threads=1)
    if form == "scalar":
        inp["A"] = workloads.draw_scalar_a(wl, seed=seed)
    elif form == "complex":
        inp["A"] = workloads.draw_complex_a(wl, seed=seed)
    return inp


def prev_token(batch, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.randn(batch, D, generator=g).to(td), torch.randn(batch, 16, generator=g).to(td)


def h0_for(batch, D, seed):
    return torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(seed)) * 0.3


def euler(form):
    return {"diagonal": jscan.prefill, "scalar": jscan.prefill_scalar_a, "complex": jscan.prefill_complex}[form]


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,dtype,with_prev", [
    (1, 1000, 512, "bf16", False),   # row-mapped kernel, ragged last tile
    (2, 300, 1024, "f32", True),     # row-mapped fp32, resumed with a previous token
    (1, 63, 128, "bf16", True),      # shorter than one tile
    (1, 1, 64, "f32", True),         # one token
    (2, 777, 40, "f32", True),       # D not a multiple of 32: lane kernel
    (3, 100, 200, "bf16", False),    # lane kernel, bf16
])
def test_matches_oracle(form, batch, L, D, dtype, with_prev):
    host = trap_case(batch, L, D, dtype, form, seed=L + D)
    h0 = h0_for(batch, D, 3) if with_prev else None
    xp, bp = prev_token(batch, D, dtype, 4) if with_prev else (None, None)
    d = to_dev(host)
    what = f"trapezoid {form} {batch}x{L}x{D} {dtype} prev={with_prev}"
    say(what)
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"],
                                   h0=None if h0 is None else h0.cuda(), x_prev=None if xp is None else xp.cuda(),
                                   B_prev=None if bp is None else bp.cuda(), form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_trapezoid(host["x"], host["delta"], host["lam"], host["A"], host["B"], host["C"],
                                            h0=h0, x_prev=xp, B_prev=bp, form=form)
    td = d["x"].dtype
    assert_parity(f64(y), y_ref, td, f"{what} y")
    assert_parity(f64(h), h_ref, td, f"{what} h_final")


@pytest.mark.parametrize("form", FORMS)
def test_prefill_4k_matches_oracle(form):
    """The 4K-token Jamba-width shape (1 x 4096 x 8192, bf16) against the full oracle."""
    host = trap_case(1, 4096, 8192, "bf16", form, seed=9)
    d = to_dev(host)
    say(f"trapezoid {form} 4K")
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_trapezoid(host["x"], host["delta"], host["lam"], host["A"], host["B"], host["C"],
                                            form=form)
    assert_parity(f64(y), y_ref, torch.bfloat16, f"trapezoid {form} 4K y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"trapezoid {form} 4K h_final")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,dtype", [(1, 1000, 512, "bf16"), (2, 777, 40, "f32")])
def test_lambda_one_is_the_euler_rule_bitwise(form, batch, L, D, dtype):
    d = to_dev(trap_case(batch, L, D, dtype, form, seed=5))
    h0 = h0_for(batch, D, 6).cuda()
    xp, bp = prev_token(batch, D, dtype, 7)
    ones = torch.ones_like(d["x"])
    y1, h1 = jscan.prefill_trapezoid(d["x"], d["delta"], ones, d["A"], d["B"], d["C"], h0=h0, x_prev=xp.cuda(),
                                     B_prev=bp.cuda(), form=form)
    y2, h2 = euler(form)(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0)
    torch.cuda.synchronize()
    assert torch.equal(bits(y1), bits(y2)) and torch.equal(bits(h1), bits(h2))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,L,D,with_prev", [(2, 200, 256, True), (1, 130, 512, False), (3, 60, 40, True)])
def test_prefill_state_equals_step_chain(form, batch, L, D, with_prev):
    d = to_dev(trap_case(batch, L, D, "bf16", form, seed=7))
    h0 = h0_for(batch, D, 4).cuda()
    if with_prev:
        xp, bp = (v.cuda() for v in prev_token(batch, D, "bf16", 8))
    else:
        xp, bp = torch.zeros_like(d["x"][:, 0]), torch.zeros_like(d["B"][:, 0])
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], h0=h0,
                                   x_prev=xp if with_prev else None, B_prev=bp if with_prev else None, form=form)
    # token rows with the previous token in front, so that every row the step reads shares one stride
    pad = lambda first, v: torch.cat([first[:, None], v], 1)  # noqa: E731
    X, Bx = pad(xp, d["x"]), pad(bp, d["B"])
    Dl, Lm, Cx = (pad(torch.zeros_like(d[k][:, 0]), d[k]) for k in ("delta", "lam", "C"))
    hs = h0.clone()
    ys = []
    for t in range(L):
        ys.append(jscan.step_trapezoid(hs, X[:, t], Bx[:, t], X[:, t + 1], Dl[:, t + 1], Lm[:, t + 1], d["A"],
                                       Bx[:, t + 1], Cx[:, t + 1], form=form).clone())
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h)), "step chain state differs from the prefill's"
    # y sums C h over the states in another order in each kernel: equal to rounding only
    assert_parity(f64(torch.stack(ys, 1)), f64(y), torch.bfloat16, f"trapezoid {form} step chain y")


@pytest.mark.parametrize("form", FORMS)
def test_resume_splits_exactly(form):
    d = to_dev(trap_case(1, 1000, 512, "bf16", form, seed=8))
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
    L1 = 320
    part = {k: (v[:, :L1].contiguous(), v[:, L1:].contiguous()) for k, v in d.items() if k != "A"}
    ya, ha = jscan.prefill_trapezoid(part["x"][0], part["delta"][0], part["lam"][0], d["A"], part["B"][0],
                                     part["C"][0], form=form)
    yb, hb = jscan.prefill_trapezoid(part["x"][1], part["delta"][1], part["lam"][1], d["A"], part["B"][1],
                                     part["C"][1], h0=ha, x_prev=d["x"][:, L1 - 1].contiguous(),
                                     B_prev=d["B"][:, L1 - 1].contiguous(), form=form)
    torch.cuda.synchronize()
    assert torch.equal(bits(torch.cat([ya, yb], 1)), bits(y)) and torch.equal(bits(hb), bits(h))


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("batch,D,dtype", [(256, 8192, "bf16"), (3, 40, "f32")])
def test_step_matches_oracle(form, batch, D, dtype):
    g = torch.Generator().manual_seed(batch + D)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    h = torch.randn(batch, D, 16, generator=g) * 0.1
    x, dl = torch.randn(batch, D, generator=g).to(td), (torch.rand(batch, D, generator=g) * 0.5).to(td)
    lam = torch.rand(batch, D, generator=g).to(td)
    xp = torch.randn(batch, D, generator=g).to(td)
    B, C, Bp = (torch.randn(batch, 16, generator=g).to(td) for _ in range(3))
    wl = workloads.Workload("adhoc_ts", 511, batch, 1, D, 16, dtype, True)
    A = {"diagonal": workloads.draw_A, "scalar": workloads.draw_scalar_a, "complex": workloads.draw_complex_a}[form](wl)
    hd = h.cuda()
    y = jscan.step_trapezoid(hd, xp.cuda(), Bp.cuda(), x.cuda(), dl.cuda(), lam.cuda(), A.cuda(), B.cuda(), C.cuda(),
                             form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.step_trapezoid(h, xp, Bp, x, dl, lam, A, B, C, form=form)
    assert_parity(f64(y), y_ref, td, f"trapezoid {form} step {batch}x{D} y")
    assert_parity(f64(hd), h_ref, td, f"trapezoid {form} step {batch}x{D} h")


@pytest.mark.parametrize("form", FORMS)
def test_prefill_64k_sampled_parity(form):
    """The 64K x 8192 workload with the trapezoidal rule, in the launch configuration the
    benchmark times, against the oracle on sampled channels over all tokens."""
    wl = workloads.get("prefill_64k")
    say(f"generating prefill_64k inputs ({form})")
    host = workloads.prefill_inputs(wl)
    host["lam"] = workloads.lam_inputs(wl)
    if form == "scalar":
        host["A"] = workloads.draw_scalar_a(wl)
    elif form == "complex":
        host["A"] = workloads.draw_complex_a(wl)
    d = to_dev(host)
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
    torch.cuda.synchronize()
    del d
    chans = sorted(set([0, 1, 31, 32, 4095, 8191] + np.random.default_rng(6).choice(wl.D, 10, replace=False).tolist()))
    say(f"oracle on {len(chans)} channels x {wl.L} tokens")
    y_ref, h_ref = oracle.prefill_trapezoid(host["x"][:, :, chans], host["delta"][:, :, chans],
                                            host["lam"][:, :, chans], host["A"][chans], host["B"], host["C"], form=form)
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, f"trapezoid {form} 64K y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, f"trapezoid {form} 64K h_final (sampled)")

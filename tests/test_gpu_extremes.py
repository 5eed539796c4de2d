"""Value regimes away from the benchmark's distributions, on the GPU against the fp64 oracle
(max|y - y_ref| <= tol * max|y_ref|, 1e-4 fp32, 2e-2 bf16), for each form of A, on the
row-mapped kernel (D a multiple of 32, ragged last tile) and the lane kernel (D = 40):

* fast forgetting: large delta times strongly negative A, so most decays underflow to zero and
  y is mostly the current token's own term;
* long memory: delta ~ 1e-4 and |A| ~ 1e-2, so every decay is within 3e-5 of one and the state
  sums thousands of inputs;
* large magnitudes: x, B and C of order 1e3, 1e2 and 1e2;
* mixed scales: delta log-uniform over five decades, token by token.

In every regime the prefill's final state equals the decode step chain bit for bit.  The
exponential-trapezoidal rule and the rank-4 MIMO scan (with and without it) run the same
regimes on the row-mapped kernels."""
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
from gpu_util import assert_parity, bits, f64, say

pytestmark = pytest.mark.gpu

FORMS = ["diagonal", "scalar", "complex"]
REGIMES = ["fast_forget", "long_memory", "large_values", "mixed_scales"]


def draw(regime, form, batch, L, D, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    u = lambda *s: torch.rand(*s, generator=g, dtype=torch.float64)  # noqa: E731
    n = lambda *s: torch.randn(*s, generator=g, dtype=torch.float64)  # noqa: E731
    x, B, C = n(batch, L, D), n(batch, L, 16), n(batch, L, 16)
    a_scale = 1.0
    if regime == "fast_forget":
        delta = torch.nn.functional.softplus(n(batch, L, D) + 3.0)
        a_scale = 4.0
    elif regime == "long_memory":
        delta = 1e-4 * (0.5 + u(batch, L, D))
        a_scale = 1e-2
    elif regime == "large_values":
        delta = torch.nn.functional.softplus(n(batch, L, D) - 2.0)
        x, B, C = 1e3 * x, 1e2 * B, 1e2 * C
    else:
        delta = 10.0 ** (-4.0 + 5.0 * u(batch, L, D))
    if form == "scalar":
        A = -a_scale * (0.5 + u(D))
    elif form == "complex":
        A = torch.empty(D, 16, dtype=torch.float64)
        A[:, 0::2] = -a_scale * torch.arange(1, 9, dtype=torch.float64)[None, :] * (0.5 + u(D, 8))
        A[:, 1::2] = torch.pi * (2.0 * u(D, 8) - 1.0)
    else:
        A = -a_scale * torch.arange(1, 17, dtype=torch.float64)[None, :] * (0.5 + u(D, 16))
    return {"x": x.to(td), "delta": delta.to(td), "A": A.float(), "B": B.to(td), "C": C.to(td)}


def run_prefill(form, d):
    fn = {"diagonal": jscan.prefill, "scalar": jscan.prefill_scalar_a, "complex": jscan.prefill_complex}[form]
    return fn(d["x"], d["delta"], d["A"], d["B"], d["C"])


def run_oracle(form, h):
    fn = {"diagonal": oracle.prefill, "scalar": oracle.prefill_scalar_a, "complex": oracle.prefill_complex}[form]
    return fn(h["x"], h["delta"], h["A"], h["B"], h["C"])


def run_step(form, hs, d, t):
    fn = {"diagonal": jscan.step, "scalar": jscan.step_scalar_a, "complex": jscan.step_complex}[form]
    return fn(hs, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t])


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("regime", REGIMES)
@pytest.mark.parametrize("batch,L,D,dtype", [(1, 700, 256, "bf16"), (2, 300, 40, "f32")])
def test_regime_matches_oracle(form, regime, batch, L, D, dtype):
    if regime == "long_memory":
        L *= 4
    host = draw(regime, form, batch, L, D, dtype, seed=100 * REGIMES.index(regime) + 10 * FORMS.index(form) + D)
    d = {k: v.cuda() for k, v in host.items()}
    what = f"{regime} {form} {batch}x{L}x{D} {dtype}"
    say(what)
    y, h = run_prefill(form, d)
    torch.cuda.synchronize()
    y_ref, h_ref = run_oracle(form, host)
    td = d["x"].dtype
    assert_parity(f64(y), y_ref, td, f"{what} y")
    assert_parity(f64(h), h_ref, td, f"{what} h_final")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("regime", REGIMES)
def test_regime_state_equals_step_chain(form, regime):
    host = draw(regime, form, 2, 90, 64, "bf16", seed=7)
    d = {k: v.cuda() for k, v in host.items()}
    _, h = run_prefill(form, d)
    hs = torch.zeros_like(h)
    for t in range(host["x"].shape[1]):
        run_step(form, hs, d, t)
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h)), f"{regime} {form}: step chain state differs from the prefill's"


def with_lam(host, seed):
    """lam in (0, 1), rows like delta."""
    g = torch.Generator().manual_seed(seed)
    return torch.rand(host["delta"].shape, generator=g).to(host["delta"].dtype)


def to_mimo(host, R, seed):
    """Rank-R x [b, L, D, R], B and C [b, L, 16, R] at the regime's scales (rank 0 is the
    single-input draw)."""
    g = torch.Generator().manual_seed(seed)
    out = dict(host)
    for k in ("x", "B", "C"):
        v = host[k].double()
        scale = float(v.abs().max()) / 4.0
        extra = torch.randn(*v.shape, R - 1, generator=g, dtype=torch.float64) * scale
        out[k] = torch.cat([v[..., None], extra], -1).to(host[k].dtype).contiguous()
    return out


@pytest.mark.parametrize("form", ["diagonal", "complex"])
@pytest.mark.parametrize("regime", REGIMES)
def test_regime_trapezoid_matches_oracle(form, regime):
    L = 2800 if regime == "long_memory" else 700
    host = draw(regime, form, 1, L, 256, "bf16", seed=300 + REGIMES.index(regime))
    host["lam"] = with_lam(host, 11)
    d = {k: v.cuda() for k, v in host.items()}
    y, h = jscan.prefill_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill_trapezoid(host["x"], host["delta"], host["lam"], host["A"], host["B"], host["C"],
                                            form=form)
    what = f"trapezoid {regime} {form}"
    assert_parity(f64(y), y_ref, torch.bfloat16, f"{what} y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"{what} h_final")


@pytest.mark.parametrize("form", ["diagonal", "complex"])
@pytest.mark.parametrize("regime", REGIMES)
@pytest.mark.parametrize("trap", [False, True])
def test_regime_mimo_matches_oracle(form, regime, trap):
    L = 1400 if regime == "long_memory" else 400
    host = to_mimo(draw(regime, form, 1, L, 256, "bf16", seed=400 + REGIMES.index(regime)), 4, 12)
    if trap:
        host["lam"] = with_lam(host, 13)
    d = {k: v.cuda() for k, v in host.items()}
    if trap:
        y, h = jscan.prefill_mimo_trapezoid(d["x"], d["delta"], d["lam"], d["A"], d["B"], d["C"], form=form)
        y_ref, h_ref = oracle.prefill_mimo_trapezoid(host["x"], host["delta"], host["lam"], host["A"], host["B"],
                                                     host["C"], form=form)
    else:
        y, h = jscan.prefill_mimo(d["x"], d["delta"], d["A"], d["B"], d["C"], form=form)
        y_ref, h_ref = oracle.prefill_mimo(host["x"], host["delta"], host["A"], host["B"], host["C"], form=form)
    torch.cuda.synchronize()
    what = f"mimo R=4 trap={trap} {regime} {form}"
    assert_parity(f64(y), y_ref, torch.bfloat16, f"{what} y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"{what} h_final")

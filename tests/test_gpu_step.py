"""jscan_step on the GPU: decode parity against the oracle, and the bit-exact agreement
of prefill's final state with L successive steps (same per-element fp32 expression, same
token order)."""
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say, to_dev

pytestmark = pytest.mark.gpu


def step_chain(d, h, t0=0, t1=None):
    """Feed tokens [t0, t1) one by one through jscan_step using strided token views."""
    t1 = d["x"].shape[1] if t1 is None else t1
    # y rows go into one preallocated tensor shaped like x, through strided views like x's
    y = torch.empty_like(d["x"])
    ys = []
    for t in range(t0, t1):
        ys.append(jscan.step(h, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t], y_t=y[:, t]))
    return ys


@pytest.mark.parametrize("name,batch,L,D,dtype", [
    ("tiny", 1, 256, 64, "f32"),
    ("ragged", 1, 1000, 512, "bf16"),
    ("batch3", 3, 130, 256, "bf16"),
    ("lane-kernel", 2, 90, 40, "f32"),
])
def test_prefill_state_equals_step_chain_bitwise(name, batch, L, D, dtype):
    inp = workloads.prefill_inputs("tiny_fp32") if name == "tiny" else workloads.small_prefill(batch, L, D, dtype)
    d = to_dev(inp)
    say(f"bit-exact {name}: {tuple(d['x'].shape)}")
    _, h_pre = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    h = torch.zeros_like(h_pre)
    ys = step_chain(d, h)
    torch.cuda.synchronize()
    assert torch.equal(bits(h), bits(h_pre)), "step chain state differs from prefill state"
    y_ref, h_ref = oracle.prefill(**inp)
    y_steps = torch.stack(ys, 1)
    assert_parity(f64(y_steps), y_ref, d["x"].dtype, f"{name} step-chain y")


def test_prefill_4k_state_equals_step_chain_bitwise():
    d = to_dev(workloads.prefill_inputs("prefill_4k"))
    _, h_pre = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    h = torch.zeros_like(h_pre)
    step_chain(d, h)
    torch.cuda.synchronize()
    assert torch.equal(bits(h), bits(h_pre))


def test_step_resumes_prefill_bitwise():
    inp = workloads.small_prefill(2, 400, 512, "bf16")
    d = to_dev(inp)
    _, h_all = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    _, h = jscan.prefill(d["x"][:, :250].contiguous(), d["delta"][:, :250].contiguous(), d["A"],
                         d["B"][:, :250].contiguous(), d["C"][:, :250].contiguous())
    step_chain(d, h, 250, 400)
    assert torch.equal(bits(h), bits(h_all))


@pytest.mark.parametrize("layers,D", [(3, 512), (28, 8192)])
def test_decode_workload_layers(layers, D):
    """Batched decode: 256 sequences, one token, each layer its own state, A and token inputs."""
    wl = workloads.get("decode_256x28")
    if D != wl.D:
        wl = workloads.Workload("decode_small", wl.wid, wl.batch, 1, D, 16, "bf16", True, layers=layers)
    worst = 0.0
    for layer in range(layers):
        inp = workloads.decode_layer_inputs(wl, layer)
        d = to_dev(inp)
        h = d["h0"].clone()
        y = jscan.step(h, d["x"], d["delta"], d["A"], d["B"], d["C"])
        torch.cuda.synchronize()
        y_ref, h_ref = oracle.step(inp["h0"], inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
        worst = max(worst, assert_parity(f64(y), y_ref, torch.bfloat16, f"decode D={D} layer {layer} y"))
        assert_parity(f64(h), h_ref, torch.bfloat16, f"decode D={D} layer {layer} h")
    say(f"decode D={D}: worst y error {worst:.3e}")


def test_step_strided_rows_and_fp32():
    inp = workloads.small_prefill(4, 8, 64, "f32")
    d = to_dev(inp)
    h0 = torch.randn(4, 64, 16, device="cuda")
    y_all = torch.empty_like(d["x"])
    h = h0.clone()
    for t in range(8):
        jscan.step(h, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t], y_t=y_all[:, t])
    y_ref, h_ref = oracle.prefill(**inp, h0=h0.cpu())
    assert_parity(f64(y_all), y_ref, torch.float32, "strided fp32 steps y")
    assert_parity(f64(h), h_ref, torch.float32, "strided fp32 steps h")


def test_step_zero_delta_keeps_state_exactly():
    h = torch.randn(2, 64, 16, device="cuda")
    h0 = h.clone()
    z = torch.zeros(2, 64, dtype=torch.bfloat16, device="cuda")
    B = torch.randn(2, 16, device="cuda").to(torch.bfloat16)
    y = jscan.step(h, torch.randn(2, 64, device="cuda").to(torch.bfloat16), z, -torch.rand(64, 16, device="cuda"), B, B)
    assert torch.equal(bits(h), bits(h0))
    ref = (B.float()[:, None, :] * h0).sum(-1)
    assert torch.allclose(y.float(), ref, rtol=1e-2, atol=1e-2)


@pytest.mark.parametrize("batch", [1, 3, 5])
def test_step_odd_batches(batch):
    """Lanes carry two batch rows; an odd batch leaves the last lane one row short."""
    wl = workloads.Workload("decode_odd", 79, batch, 1, 96, 16, "bf16", True, layers=1)
    inp = workloads.decode_layer_inputs(wl, 0)
    d = to_dev(inp)
    h = d["h0"].clone()
    y = jscan.step(h, d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_ref, h_ref = oracle.step(inp["h0"], inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"])
    assert_parity(f64(y), y_ref, torch.bfloat16, f"odd batch {batch} y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"odd batch {batch} h")


def test_step_output_row_stride_is_its_own():
    """y_t's row stride (ld_y) is independent of x_t's: strided token views of x written to a
    new contiguous [batch, D], to token views of a [batch, L, D] output, and to the first D
    columns of a wider NaN-filled buffer give the same bits, and nothing past the D columns is
    written.  Checked for the single-input step, the trapezoidal step and the MIMO step."""
    batch, L, D, R = 3, 6, 256, 4
    d = to_dev(workloads.small_prefill(batch, L, D, "bf16", seed=5))
    A = d["A"]
    h_runs = [torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(2)).cuda() for _ in range(3)]
    y_tok = torch.empty_like(d["x"])
    wide = torch.full((batch, D + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    for t in range(L):
        args = (d["x"][:, t], d["delta"][:, t], A, d["B"][:, t], d["C"][:, t])
        y_new = jscan.step(h_runs[0], *args)
        jscan.step(h_runs[1], *args, y_t=y_tok[:, t])
        jscan.step(h_runs[2], *args, y_t=wide[:, :D])
        assert y_new.is_contiguous() and y_new.shape == (batch, D)
        assert torch.equal(bits(y_new), bits(y_tok[:, t])) and torch.equal(bits(y_new), bits(wide[:, :D]))
        assert torch.isnan(wide[:, D:].float()).all(), "step wrote past y_t's rows"
    assert torch.equal(bits(h_runs[0]), bits(h_runs[1])) and torch.equal(bits(h_runs[0]), bits(h_runs[2]))

    # the trapezoidal step shares the launch: token views in, contiguous and wide out
    lam = torch.rand(batch, L, D, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).cuda()
    hs = [torch.zeros(batch, D, 16, device="cuda") for _ in range(2)]
    for t in range(1, L):
        targs = (d["x"][:, t - 1], d["B"][:, t - 1], d["x"][:, t], d["delta"][:, t], lam[:, t], A, d["B"][:, t],
                 d["C"][:, t])
        y_new = jscan.step_trapezoid(hs[0], *targs)
        jscan.step_trapezoid(hs[1], *targs, y_t=wide[:, :D])
        assert torch.equal(bits(y_new), bits(wide[:, :D])) and torch.isnan(wide[:, D:].float()).all()
    assert torch.equal(bits(hs[0]), bits(hs[1]))

    # MIMO: x_t rows of D * R, y_t rows of D * R with a stride of their own
    xm = torch.randn(batch, L, D, R, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16).cuda()
    Bm = torch.randn(batch, L, 16, R, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    wide_m = torch.full((batch, D * R + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    hm = [torch.zeros(batch, D, 16, device="cuda") for _ in range(2)]
    for t in range(L):
        margs = (xm[:, t], d["delta"][:, t], A, Bm[:, t], Bm[:, t])
        y_new = jscan.step_mimo(hm[0], *margs)
        y_w = jscan.step_mimo(hm[1], *margs, y_t=wide_m[:, :D * R].view(batch, D, R))
        assert y_new.is_contiguous() and torch.equal(bits(y_new), bits(y_w))
        assert torch.isnan(wide_m[:, D * R:].float()).all(), "MIMO step wrote past y_t's rows"
    assert torch.equal(bits(hm[0]), bits(hm[1]))

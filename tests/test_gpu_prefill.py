"""jscan_prefill / jscan_prefill_resume on the GPU against the fp64 oracle, plus exact
invariants that need no oracle.  Tolerance: max|y - y_ref| <= tol * max|y_ref| with tol
1e-4 for fp32 inputs and 2e-2 for bf16 inputs (fp32 state)."""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import GlobalRel, assert_parity, bits, channel_blocks, f64, say, to_dev

pytestmark = pytest.mark.gpu


def run_case(inp, what, h0=None):
    dev = to_dev(inp)
    dtype = dev["x"].dtype
    say(f"case {what}: x {tuple(dev['x'].shape)} {dtype}")
    h0d = None if h0 is None else h0.cuda()
    y, h = jscan.prefill(dev["x"], dev["delta"], dev["A"], dev["B"], dev["C"], h0=h0d)
    torch.cuda.synchronize()
    y_ref, h_ref = oracle.prefill(inp["x"], inp["delta"], inp["A"], inp["B"], inp["C"], h0=h0)
    assert_parity(f64(y), y_ref, dtype, f"{what} y")
    assert_parity(f64(h), h_ref, dtype, f"{what} h_final")
    return y, h


def test_tiny_fp32_workload():
    run_case(workloads.prefill_inputs("tiny_fp32"), "tiny_fp32 (1x256x64)")


@pytest.mark.parametrize("batch,L,D,dtype", [
    (1, 1000, 512, "bf16"),      # rows kernel, ragged last tile
    (1, 64, 32, "bf16"),         # one block, one whole tile
    (1, 1, 64, "bf16"),          # single token
    (1, 65, 96, "f32"),          # rows kernel fp32, one token past a tile
    (2, 300, 1024, "bf16"),      # batch > 1 through the rows kernel
    (1, 130, 72, "bf16"),        # D not a multiple of 32: lane kernel
    (3, 77, 8, "f32"),           # smallest D, lane kernel
    (17, 40, 4096, "bf16"),      # batch * D above 65536: still the rows kernel
])
def test_prefill_shapes(batch, L, D, dtype):
    run_case(workloads.small_prefill(batch, L, D, dtype), f"{batch}x{L}x{D} {dtype}")


def test_resume_from_state():
    inp = workloads.small_prefill(2, 200, 256, "bf16")
    h0 = torch.from_numpy(np.random.default_rng(3).normal(0, 0.5, size=(2, 256, 16)).astype(np.float32))
    run_case(inp, "resume 2x200x256", h0=h0)


def test_prefill_4k_workload():
    """The 4K-token Jamba-layer prefill (batch 1, D 8192) against the full oracle."""
    run_case(workloads.prefill_inputs("prefill_4k"), "prefill_4k (1x4096x8192)")


def _dev_small(seed=0, batch=1, L=333, D=256, dtype="bf16"):
    return to_dev(workloads.small_prefill(batch, L, D, dtype, seed=seed))


def test_split_resume_is_bit_identical():
    d = _dev_small(L=1000, D=512)
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    for cut in (1, 64, 333, 999):
        y1, h1 = jscan.prefill(d["x"][:, :cut].contiguous(), d["delta"][:, :cut].contiguous(), d["A"],
                               d["B"][:, :cut].contiguous(), d["C"][:, :cut].contiguous())
        y2, h2 = jscan.prefill(d["x"][:, cut:].contiguous(), d["delta"][:, cut:].contiguous(), d["A"],
                               d["B"][:, cut:].contiguous(), d["C"][:, cut:].contiguous(), h0=h1)
        assert torch.equal(bits(h2), bits(h)), f"cut {cut}: state differs"
        assert torch.equal(bits(torch.cat([y1, y2], 1)), bits(y)), f"cut {cut}: y differs"
    # in place: h0 is h_final
    hs = torch.zeros_like(h)
    jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=hs, h_final=hs)
    assert torch.equal(bits(hs), bits(h))


def test_deterministic():
    d = _dev_small(L=700, D=1024)
    y1, h1 = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y2, h2 = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    assert torch.equal(bits(y1), bits(y2)) and torch.equal(bits(h1), bits(h2))


def test_exact_scaling_and_sign():
    d = _dev_small(L=200, D=256)
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y2, h2 = jscan.prefill(2 * d["x"], d["delta"], d["A"], d["B"], d["C"])
    assert torch.equal(bits(y2), bits(2 * y)) and torch.equal(bits(h2), bits(2 * h))
    yb, hb = jscan.prefill(d["x"], d["delta"], d["A"], 2 * d["B"], d["C"])
    assert torch.equal(bits(yb), bits(2 * y)) and torch.equal(bits(hb), bits(2 * h))
    yn, hn = jscan.prefill(-d["x"], d["delta"], d["A"], d["B"], d["C"])
    # A sum that cancels exactly is +0 whatever the signs of its terms (round to nearest), so
    # where y is exactly zero, y(-x) is +0 too, not -0: y is compared by value there.
    nz = y != 0
    assert torch.equal(yn, -y) and torch.equal(bits(yn[nz]), bits(-y[nz]))
    assert torch.equal(bits(hn), bits(-h))
    yc, hc = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], 2 * d["C"])
    assert torch.equal(bits(yc), bits(2 * y)) and torch.equal(bits(hc), bits(h))


def test_causality():
    d = _dev_small(L=300, D=256)
    y, _ = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    t0 = 150
    x2, d2, C2 = d["x"].clone(), d["delta"].clone(), d["C"].clone()
    x2[:, t0 + 1:] = torch.randn_like(x2[:, t0 + 1:])
    d2[:, t0 + 1:] = 2.0
    C2[:, t0 + 1:] += 1
    y2, _ = jscan.prefill(x2, d2, d["A"], d["B"], C2)
    assert torch.equal(bits(y2[:, :t0 + 1]), bits(y[:, :t0 + 1]))
    assert not torch.equal(bits(y2[:, t0 + 1:]), bits(y[:, t0 + 1:]))


def test_channel_permutation():
    d = _dev_small(L=200, D=512)
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    perm = torch.from_numpy(np.random.default_rng(5).permutation(512)).cuda()
    yp, hp = jscan.prefill(d["x"][:, :, perm].contiguous(), d["delta"][:, :, perm].contiguous(),
                           d["A"][perm].contiguous(), d["B"], d["C"])
    assert torch.equal(bits(yp), bits(y[:, :, perm].contiguous())) and torch.equal(bits(hp), bits(h[:, perm].contiguous()))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_zero_A_prefix_sum_is_exact(dtype):
    """A = 0, delta = 0.5, B = 2, x = 1, C = 1: every input term is 1, so h_t = t + 1 and
    y_t = 16 (t + 1), exactly (v_exp_f32(0) = 1)."""
    L, D = 3000, 64
    x = torch.ones(1, L, D, dtype=dtype, device="cuda")
    dl = torch.full((1, L, D), 0.5, dtype=dtype, device="cuda")
    A = torch.zeros(D, 16, device="cuda")
    B = torch.full((1, L, 16), 2.0, dtype=dtype, device="cuda")
    C = torch.ones(1, L, 16, dtype=dtype, device="cuda")
    y, h = jscan.prefill(x, dl, A, B, C)
    t1 = torch.arange(1, L + 1, dtype=torch.float64, device="cuda")
    assert torch.equal(h, torch.full_like(h, float(L)))
    expect = (16 * t1).to(torch.float32).to(dtype)[None, :, None].expand(1, L, D)
    assert torch.equal(bits(y), bits(expect.contiguous()))


def test_zero_delta_freezes_state():
    d = _dev_small(L=100, D=128)
    h0 = torch.randn(1, 128, 16, device="cuda")
    y, h = jscan.prefill(d["x"], torch.zeros_like(d["delta"]), d["A"], d["B"], d["C"], h0=h0)
    assert torch.equal(bits(h), bits(h0))


def test_empty_sequence():
    d = _dev_small(L=10, D=64)
    e = lambda t: t[:, :0].contiguous()  # noqa: E731
    h0 = torch.randn(1, 64, 16, device="cuda")
    y, h = jscan.prefill(e(d["x"]), e(d["delta"]), d["A"], e(d["B"]), e(d["C"]))
    assert y.shape == (1, 0, 64) and torch.equal(h, torch.zeros_like(h))
    y, h = jscan.prefill(e(d["x"]), e(d["delta"]), d["A"], e(d["B"]), e(d["C"]), h0=h0)
    assert torch.equal(h, h0)


def test_nan_poisoned_outputs_are_overwritten():
    d = _dev_small(L=321, D=256)
    y = torch.full_like(d["x"], float("nan"))
    h = torch.full((1, 256, 16), float("nan"), device="cuda")
    jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y, h_final=h)
    assert torch.isfinite(y.float()).all() and torch.isfinite(h).all()


def test_api_errors_raise():
    d = _dev_small(L=64, D=64)
    with pytest.raises(ValueError):
        jscan.prefill(d["x"], d["delta"], d["A"], d["B"][:, :, :8], d["C"])
    with pytest.raises(jscan.JScanError) as ei:
        jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=d["x"])   # y aliases x
    assert ei.value.status == 5


@pytest.mark.timeout(600)
def test_batched_prefill_every_channel():
    """Sixteen 4K-token prompts at D = 8192 (a batched prefill: 131072 channels, run by the
    row-mapped kernel) against the oracle on every channel of every sequence, streamed one
    block of channels at a time."""
    inp = workloads.small_prefill(16, 4096, 8192, "bf16", seed=21)
    d = to_dev(inp)
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    y_host, h_host = y.cpu(), h.cpu()
    gy, gh = GlobalRel("16x4096x8192 y"), GlobalRel("16x4096x8192 h_final")
    for c0, c1 in channel_blocks(8192, 1024):
        y_ref, h_ref = oracle.prefill(inp["x"][:, :, c0:c1], inp["delta"][:, :, c0:c1], inp["A"][c0:c1], inp["B"],
                                      inp["C"], nthreads=16)
        gy.add(f64(y_host[:, :, c0:c1]), y_ref)
        gh.add(f64(h_host[:, c0:c1]), h_ref)
    gy.check(torch.bfloat16)
    gh.check(torch.bfloat16)

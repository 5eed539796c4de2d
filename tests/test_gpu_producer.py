"""jscan_ssm_inputs (the producer side: delta, B and C from x) on the GPU against the fp64
oracle in oracle/producer.py.

Every output is one rounding of an fp32 value to bf16.  The fp32 value differs from the
oracle's fp64 value only by accumulation and function rounding, so the two bf16 results are
equal or one bf16 step apart (when the values straddle a rounding boundary).  The test allows
one step, |gpu - ref| <= 2^-7 |ref|, element by element, plus an absolute 2^-16 of the
tensor's largest value: a dot product's fp32 error scales with its terms, not its result, so
an output that cancels to near zero can miss by more than a step of its own tiny size.  That
slack is still 500 times below a bf16 step at the tensor's scale.  delta is checked from the
GPU's own d_low, so a step in d_low does not carry into delta's check.
"""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_bf16_sums_close, assert_parity, bits, f64, say
from oracle import producer as P

pytestmark = pytest.mark.gpu

EPS = 1e-6


def one_step_close(got, ref, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = 2.0 ** -7 * np.maximum(np.abs(ref), np.abs(got)) + 2.0 ** -16 * np.max(np.abs(ref))
    bad = np.abs(got - ref) > bound
    differ = np.count_nonzero(got != ref)
    say(f"{what}: {differ} of {ref.size} elements one bf16 step apart, {np.count_nonzero(bad)} beyond")
    assert not bad.any(), f"{what}: {np.count_nonzero(bad)} elements beyond one bf16 step"
    assert differ <= max(8, ref.size // 200), f"{what}: too many rounding differences ({differ})"


def delta_end_to_end_close(delta, d_low, d_low_ref, wts, what):
    """The GPU's delta against the oracle's own end-to-end delta (computed from the oracle's
    d_low, not the GPU's).  Where the two d_low differ by a bf16 step, delta's pre-activation
    W_dt d_low + b_dt moves by at most sum_k |W_dt[d, k]| |d_low[k] - d_low_ref[k]|, and
    softplus moves by no more than its argument (its slope is below 1).  On top of that each
    side rounds delta once to bf16 (together at most one bf16 step) and accumulates in fp32
    (the 2^-16 slack of one_step_close)."""
    delta = np.asarray(delta, np.float64)
    w = np.abs(wts["w_dt"].double().numpy())
    ref = P.delta_from_low(d_low_ref, wts["w_dt"].double().numpy(), wts["b_dt"].numpy())
    moved = np.abs(np.asarray(d_low, np.float64) - d_low_ref) @ w.T
    bound = 2.0 ** -7 * np.maximum(np.abs(ref), np.abs(delta)) + moved + 2.0 ** -16 * np.max(np.abs(ref))
    bad = np.abs(delta - ref) > bound
    say(f"{what} (end to end): {np.count_nonzero(delta != ref)} of {ref.size} elements differ, "
        f"{np.count_nonzero(bad)} beyond the bound")
    assert not bad.any(), f"{what}: {np.count_nonzero(bad)} elements beyond the end-to-end bound"
    assert np.all(delta > 0) and np.all(np.isfinite(delta))


def run(M, D, R, seed=0, rows=None):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(M, D, generator=g).to(torch.bfloat16)
    wts = workloads.producer_weights(D, R, seed=seed)
    dev = {k: v.cuda() for k, v in wts.items()}
    xd = x.cuda()
    delta, B, C, d_low = jscan.ssm_inputs(xd, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"],
                                          dev["b_dt"], eps=EPS)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    xs = x[sel].double().numpy()
    d_ref, B_ref, C_ref, _ = P.ssm_inputs(xs, wts["w_x"].double().numpy(), wts["g_d"].numpy(), wts["g_b"].numpy(),
                                          wts["g_c"].numpy(), wts["w_dt"].double().numpy(), wts["b_dt"].numpy(), EPS, R)
    tag = f"{M}x{D} R={R}"
    one_step_close(f64(d_low)[sel], d_ref, f"{tag} d_low")
    one_step_close(f64(B)[sel], B_ref, f"{tag} B")
    one_step_close(f64(C)[sel], C_ref, f"{tag} C")
    delta_end_to_end_close(f64(delta)[sel], f64(d_low)[sel], d_ref, wts, f"{tag} delta")
    delta_ref = P.delta_from_low(f64(d_low)[sel], wts["w_dt"].double().numpy(), wts["b_dt"].numpy())
    one_step_close(f64(delta)[sel], delta_ref, f"{tag} delta (staged: from the GPU's d_low)")
    return x, wts, (delta, B, C, d_low)


@pytest.mark.parametrize("M,D,R", [
    (256, 256, 64),      # one whole x-projection row tile; half of one delta channel slice
    (1000, 512, 128),    # ragged last row tile
    (777, 1024, 256),    # the full rank, ragged
    (1, 128, 256),       # a single token (decode-sized)
    (300, 640, 256),     # a partial last delta channel slice (128 of 512 channels) and ragged tokens
    (20007, 384, 64),    # about five token tiles per group, six of eight channel waves busy, ragged
    (700, 8192, 256),    # two or three token tiles per group (the pipeline's short-group waits), ragged
    (1500, 8192, 64),    # five or six token tiles per group at the smallest rank, ragged
])
def test_ssm_inputs_match_oracle(M, D, R):
    run(M, D, R, seed=M + D)


def test_ssm_inputs_deterministic():
    x = torch.randn(513, 512, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
    w = {k: v.cuda() for k, v in workloads.producer_weights(512, 128).items()}
    a = jscan.ssm_inputs(x, w["w_x"], w["g_d"], w["g_b"], w["g_c"], w["w_dt"], w["b_dt"])
    b = jscan.ssm_inputs(x, w["w_x"], w["g_d"], w["g_b"], w["g_c"], w["w_dt"], w["b_dt"])
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(bits(u), bits(v))


def test_producer_then_scan_against_oracle():
    """x -> (delta, B, C) -> scan, end to end, against the oracle doing the same two stages
    (the oracle scan is fed the oracle's own bf16 delta, B and C)."""
    L, D, R = 1024, 512, 256
    inp = workloads.small_prefill(1, L, D, "bf16", seed=12)
    wts = workloads.producer_weights(D, R, seed=12)
    dev = {k: v.cuda() for k, v in wts.items()}
    x = inp["x"].cuda()
    delta, B, C, _ = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"])
    A = inp["A"].cuda()
    y, h = jscan.prefill(x, delta, A, B, C)
    torch.cuda.synchronize()
    d_ref, B_ref, C_ref, delta_ref = P.ssm_inputs(inp["x"][0].double().numpy(), wts["w_x"].double().numpy(),
                                                  wts["g_d"].numpy(), wts["g_b"].numpy(), wts["g_c"].numpy(),
                                                  wts["w_dt"].double().numpy(), wts["b_dt"].numpy(), 1e-6, R)
    y_ref, h_ref = oracle.prefill(inp["x"].double().numpy(), delta_ref[None], inp["A"].double().numpy(), B_ref[None],
                                  C_ref[None])
    assert_parity(f64(y), y_ref, torch.bfloat16, "producer + scan y")
    assert_parity(f64(h), h_ref, torch.bfloat16, "producer + scan h_final")


def test_ssm_inputs_full_size_sampled_rows():
    """The 64K x 8192 workload's x through the producer at full size (R = 256), checked on
    sampled rows (rows are independent): the first and last rows of row tiles and random ones."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k x")
    x = workloads.prefill_inputs(wl)["x"][0]
    wts = workloads.producer_weights(wl.D, 256)
    dev = {k: v.cuda() for k, v in wts.items()}
    delta, B, C, d_low = jscan.ssm_inputs(x.cuda(), dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"],
                                          dev["b_dt"])
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 127, 128, 129, 4095, 32768, 65535] +
                      np.random.default_rng(3).choice(wl.L, 24, replace=False).tolist()))
    idx = torch.tensor(rows)
    xs = x[idx].double().numpy()
    d_ref, B_ref, C_ref, _ = P.ssm_inputs(xs, wts["w_x"].double().numpy(), wts["g_d"].numpy(), wts["g_b"].numpy(),
                                          wts["g_c"].numpy(), wts["w_dt"].double().numpy(), wts["b_dt"].numpy(), EPS,
                                          256)
    dl = f64(d_low.cpu()[idx])
    one_step_close(dl, d_ref, "64K d_low (sampled rows)")
    one_step_close(f64(B.cpu()[idx]), B_ref, "64K B (sampled rows)")
    one_step_close(f64(C.cpu()[idx]), C_ref, "64K C (sampled rows)")
    delta_end_to_end_close(f64(delta.cpu()[idx]), dl, d_ref, wts, "64K delta (sampled rows)")
    one_step_close(f64(delta.cpu()[idx]), P.delta_from_low(dl, wts["w_dt"].double().numpy(), wts["b_dt"].numpy()),
                   "64K delta (sampled rows, staged: from the GPU's d_low)")
    assert torch.isfinite(delta.float()).all() and float(delta.float().min()) > 0


@pytest.mark.parametrize("batch,L,D,with_h0", [(1, 1000, 512, False), (2, 300, 1024, True), (1, 4096, 8192, False),
                                                (1, 63, 128, True), (1, 1, 128, False)])
def test_fused_prefill_is_bit_identical_to_producer_then_scan(batch, L, D, with_h0):
    """Delta computed inside the scan (jscan_prefill_fused) equals the producer's delta bit for
    bit, so h_final matches jscan_ssm_inputs followed by jscan_prefill(_resume) exactly.  y sums
    over the states differently on the matrix cores (the fused scan sums the lanes' partials,
    rounded to bf16; the plain scan contracts the states, rounded to bf16, with C), so y agrees to
    those roundings."""
    inp = workloads.small_prefill(batch, L, D, "bf16", seed=L + D)
    wts = workloads.producer_weights(D, 256, seed=D)
    dev = {k: v.cuda() for k, v in wts.items()}
    x = inp["x"].cuda()
    A = inp["A"].cuda()
    h0 = (torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(1)) * 0.1).cuda() if with_h0 else None
    delta, B, C, d_low = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"])
    y1, h1 = jscan.prefill(x, delta, A, B, C, h0=h0)
    _, B2, C2, d_low2 = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"],
                                         skip_delta=True)
    y2, h2 = jscan.prefill_fused(x, d_low2, dev["w_dt"], dev["b_dt"], A, B2, C2, h0=h0)
    torch.cuda.synchronize()
    say(f"fused {batch}x{L}x{D} h0={with_h0}")
    assert torch.equal(bits(d_low), bits(d_low2)) and torch.equal(bits(B), bits(B2))
    assert torch.equal(bits(h1), bits(h2)), "fused h_final differs"
    assert_bf16_sums_close(y1, y2, "fused y")


def test_fused_prefill_64k_full_size():
    """The 64K x 8192 workload through the producer in the launch configurations the
    benchmark times: the fused scan (delta computed on the load path) equals the producer's
    stored delta followed by jscan_prefill on every state bit, and on y to the roundings of
    the two sums over states."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k x, A")
    inp = workloads.prefill_inputs(wl)
    wts = workloads.producer_weights(wl.D, 256)
    dev = {k: v.cuda() for k, v in wts.items()}
    x, A = inp["x"].cuda(), inp["A"].cuda()
    del inp
    delta, B, C, d_low = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"])
    y1, h1 = jscan.prefill(x, delta, A, B, C)
    del delta
    y2, h2 = jscan.prefill_fused(x, d_low, dev["w_dt"], dev["b_dt"], A, B, C)
    torch.cuda.synchronize()
    assert torch.equal(h1.view(torch.int32), h2.view(torch.int32)), "fused 64K h_final differs"
    for i in range(0, wl.L, 8192):   # in token blocks, to bound the fp64 copies
        assert_bf16_sums_close(y1[:, i:i + 8192], y2[:, i:i + 8192], f"fused 64K y, tokens {i}..")


def oracle_producer_then_scan(x, wts, A, h0=None, R=256):
    """The oracle's x -> (delta, B, C) (oracle.producer) -> scan (oracle.prefill), fed nothing
    the GPU computed.  x [batch, L, D] bf16."""
    batch, L, D = x.shape
    ds, Bs, Cs = [], [], []
    for b in range(batch):
        _, B_ref, C_ref, delta_ref = P.ssm_inputs(x[b].double().numpy(), wts["w_x"].double().numpy(),
                                                  wts["g_d"].numpy(), wts["g_b"].numpy(), wts["g_c"].numpy(),
                                                  wts["w_dt"].double().numpy(), wts["b_dt"].numpy(), EPS, R)
        ds.append(delta_ref)
        Bs.append(B_ref)
        Cs.append(C_ref)
    return oracle.prefill(x.double().numpy(), np.stack(ds), A.double().numpy(), np.stack(Bs), np.stack(Cs),
                          h0=None if h0 is None else h0.double().numpy(), nthreads=16)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("batch,L,D,with_h0", [(1, 4096, 8192, False), (2, 300, 1024, True), (1, 63, 128, True)])
def test_fused_prefill_against_oracle(batch, L, D, with_h0):
    """x -> jscan_ssm_inputs (x projection only) -> jscan_prefill_fused (delta's projection,
    bias and softplus inside the scan) against the oracle's producer followed by the oracle's
    scan on the same x, at the bf16 tolerance."""
    inp = workloads.small_prefill(batch, L, D, "bf16", seed=L + 3 * D)
    wts = workloads.producer_weights(D, 256, seed=D + 1)
    dev = {k: v.cuda() for k, v in wts.items()}
    x, A = inp["x"].cuda(), inp["A"].cuda()
    h0 = (torch.randn(batch, D, 16, generator=torch.Generator().manual_seed(2)) * 0.1) if with_h0 else None
    _, B, C, d_low = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"],
                                      eps=EPS, skip_delta=True)
    y, h = jscan.prefill_fused(x, d_low, dev["w_dt"], dev["b_dt"], A, B, C, h0=None if h0 is None else h0.cuda())
    torch.cuda.synchronize()
    say(f"fused {batch}x{L}x{D} h0={with_h0} against the oracle's producer + scan")
    y_ref, h_ref = oracle_producer_then_scan(inp["x"], wts, inp["A"], h0)
    assert_parity(f64(y), y_ref, torch.bfloat16, f"fused {batch}x{L}x{D} y")
    assert_parity(f64(h), h_ref, torch.bfloat16, f"fused {batch}x{L}x{D} h_final")


@pytest.mark.timeout(900)
def test_fused_prefill_64k_against_oracle_sampled_channels():
    """The 64K x 8192 workload's x through the x projection and the fused scan, in the launch
    configuration the benchmark times (bench.py --producer --fused), against the oracle's
    producer and scan: the oracle projects every token (B and C are shared by all channels)
    and scans sampled channels over all 65536 tokens."""
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k x, A")
    inp = workloads.prefill_inputs(wl)
    wts = workloads.producer_weights(wl.D, 256)
    dev = {k: v.cuda() for k, v in wts.items()}
    x, A = inp["x"].cuda(), inp["A"].cuda()
    _, B, C, d_low = jscan.ssm_inputs(x, dev["w_x"], dev["g_d"], dev["g_b"], dev["g_c"], dev["w_dt"], dev["b_dt"],
                                      eps=EPS, skip_delta=True)
    y, h = jscan.prefill_fused(x, d_low, dev["w_dt"], dev["b_dt"], A, B, C)
    torch.cuda.synchronize()
    chans = sorted(set([0, 1, 15, 16, 31, 32, 4095, 4096, 8190, 8191] +
                       np.random.default_rng(4).choice(wl.D, 14, replace=False).tolist()))
    say("oracle producer over 65536 tokens")
    dl_ref, B_ref, C_ref = P.ssm_inputs_low(inp["x"][0].double().numpy(), wts["w_x"].double().numpy(),
                                            wts["g_d"].numpy(), wts["g_b"].numpy(), wts["g_c"].numpy(), EPS, 256)
    delta_ref = P.delta_from_low(dl_ref, wts["w_dt"][chans].double().numpy(), wts["b_dt"][chans].numpy())
    say(f"oracle scan on {len(chans)} channels x {wl.L} tokens")
    y_ref, h_ref = oracle.prefill(inp["x"][:, :, chans], delta_ref[None], inp["A"][chans], B_ref[None], C_ref[None],
                                  nthreads=16)
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, "fused 64K y (sampled channels)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, "fused 64K h_final (sampled channels)")

"""Full-size long-context workloads on the GPU, in the launch configuration the bench times.

The oracle cannot redo a whole 64K x 8192 or 256K x 8192 scan in seconds, but channels are
independent, so it recomputes a sample of channels over the whole sequence: channels at
the edges of the 16-channel lane groups, the 32-channel workgroups and the XCD channel
ranges, plus random ones.  The tolerance is the workload's own, taken against the sampled
max|y_ref| (which can only make the check stricter than against the global maximum).
"""
import numpy as np
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import oracle
import workloads
from gpu_util import assert_parity, bits, f64, say

pytestmark = pytest.mark.gpu


_INPUTS = {}


def inputs_256k():
    """Host inputs of the 256K workload (+64 tokens), generated once per test module."""
    if "256k" not in _INPUTS:
        wl = workloads.get("prefill_256k")
        say("generating prefill_256k inputs (+64 tokens)")
        _INPUTS["256k"] = workloads.prefill_inputs(wl, t1=wl.L + wl.extra_tokens)
    return _INPUTS["256k"]


def sample_channels(D, seed=0):
    edges = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 1023, 1024, D // 2 - 1, D // 2, D - 33, D - 32, D - 2, D - 1]
    rnd = np.random.default_rng(seed).choice(D, 14, replace=False).tolist()
    return sorted(set(e for e in edges + rnd if 0 <= e < D))


def oracle_on_channels(inp, chans, t1=None):
    t1 = inp["x"].shape[1] if t1 is None else t1
    x = inp["x"][:, :t1, chans]
    dl = inp["delta"][:, :t1, chans]
    return oracle.prefill(x, dl, inp["A"][chans], inp["B"][:, :t1], inp["C"][:, :t1])


def step_chain(d, h, t0, t1):
    ys = []
    for t in range(t0, t1):
        ys.append(jscan.step(h, d["x"][:, t], d["delta"][:, t], d["A"], d["B"][:, t], d["C"][:, t]))
    return ys


def test_prefill_64k_sampled_parity_and_bit_exact_steps():
    wl = workloads.get("prefill_64k")
    say("generating prefill_64k inputs")
    inp = workloads.prefill_inputs(wl)
    d = {k: v.cuda() for k, v in inp.items()}
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    torch.cuda.synchronize()
    chans = sample_channels(wl.D)
    say(f"oracle on {len(chans)} channels x {wl.L} tokens")
    y_ref, h_ref = oracle_on_channels(inp, chans)
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref, torch.bfloat16, "prefill_64k y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref, torch.bfloat16, "prefill_64k h_final (sampled)")
    assert torch.isfinite(y.float()).all()
    say("65536 decode steps from the zero state")
    hs = torch.zeros_like(h)
    step_chain(d, hs, 0, wl.L)
    torch.cuda.synchronize()
    assert torch.equal(bits(hs), bits(h)), "step chain final state differs from prefill (64K)"


def test_prefill_256k_sampled_parity_and_step_continuation():
    """256K tokens through prefill, then 64 more tokens through jscan_step from the GPU's own
    final state; the oracle continues its fp64 state over the same 64 tokens."""
    wl = workloads.get("prefill_256k")
    inp = inputs_256k()
    d = {k: v.cuda() for k, v in inp.items()}
    L = wl.L
    pre = {k: (v if k == "A" else v[:, :L]) for k, v in d.items()}
    y, h = jscan.prefill(pre["x"], pre["delta"], pre["A"], pre["B"], pre["C"])
    torch.cuda.synchronize()
    chans = sample_channels(wl.D, seed=1)
    say(f"oracle on {len(chans)} channels x {L + wl.extra_tokens} tokens")
    y_ref_all, h_ref_all = oracle_on_channels(inp, chans)          # all L + 64 tokens
    _, h_ref_L = oracle_on_channels(inp, chans, t1=L)
    idx = torch.tensor(chans, device="cuda")
    assert_parity(f64(y.index_select(2, idx)), y_ref_all[:, :L], torch.bfloat16, "prefill_256k y (sampled)")
    assert_parity(f64(h.index_select(1, idx)), h_ref_L, torch.bfloat16, "prefill_256k h_final (sampled)")
    ys = step_chain(d, h, L, L + wl.extra_tokens)
    y_steps = torch.stack(ys, 1)
    torch.cuda.synchronize()
    assert_parity(f64(y_steps.index_select(2, idx)), y_ref_all[:, L:], torch.bfloat16, "256k + 64 step outputs")
    assert_parity(f64(h.index_select(1, idx)), h_ref_all, torch.bfloat16, "state after 256k + 64 tokens")


def test_prefill_256k_matches_resume_split():
    """The same 256K scan split at 100,000 tokens and resumed gives identical bits (the x
    array here is 4 GiB, so this also covers offsets past 2^31 elements)."""
    wl = workloads.get("prefill_256k")
    full = inputs_256k()
    d = {k: (v if k == "A" else v[:, :wl.L]).cuda() for k, v in full.items()}
    y, h = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    cut = 100_000
    part = lambda v, a, b: v[:, a:b].contiguous()  # noqa: E731
    y1, h1 = jscan.prefill(part(d["x"], 0, cut), part(d["delta"], 0, cut), d["A"], part(d["B"], 0, cut),
                           part(d["C"], 0, cut))
    y2, h2 = jscan.prefill(part(d["x"], cut, None), part(d["delta"], cut, None), d["A"], part(d["B"], cut, None),
                           part(d["C"], cut, None), h0=h1)
    assert torch.equal(bits(h2), bits(h))
    assert torch.equal(bits(y1), bits(y[:, :cut].contiguous())) and torch.equal(bits(y2), bits(y[:, cut:].contiguous()))

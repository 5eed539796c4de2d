"""Helpers shared by the GPU parity tests."""
import sys

import numpy as np
import torch

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}   # max|y - y_ref| <= tol * max|y_ref|


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


def to_dev(inp, dev="cuda"):
    return {k: v.to(dev) for k, v in inp.items()}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def global_rel(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref)) / max(np.max(np.abs(ref)), 1e-30))


def assert_parity(got, ref, dtype, what):
    err = global_rel(got, ref)
    say(f"{what}: max|err|/max|ref| = {err:.3e} (tol {TOL[dtype]:g})")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert err <= TOL[dtype], f"{what}: {err:.3e} > {TOL[dtype]:g}"
    return err


def bits(t):
    return t.detach().contiguous().view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu()


class GlobalRel:
    """max|got - ref| / max|ref| accumulated over blocks of one output, so that a whole tensor
    can be compared without holding its fp64 reference at once."""

    def __init__(self, what):
        self.what, self.err, self.ref, self.finite = what, 0.0, 0.0, True

    def add(self, got, ref):
        got = np.asarray(got, np.float64)
        ref = np.asarray(ref, np.float64)
        self.finite = self.finite and bool(np.all(np.isfinite(got)))
        self.err = max(self.err, float(np.max(np.abs(got - ref))))
        self.ref = max(self.ref, float(np.max(np.abs(ref))))

    def check(self, dtype):
        rel = self.err / max(self.ref, 1e-30)
        say(f"{self.what}: max|err|/max|ref| = {rel:.3e} over every element (tol {TOL[dtype]:g})")
        assert self.finite, f"{self.what}: non-finite output"
        assert rel <= TOL[dtype], f"{self.what}: {rel:.3e} > {TOL[dtype]:g}"
        return rel


def channel_blocks(D, block):
    return [(c0, min(c0 + block, D)) for c0 in range(0, D, block)]


def assert_bf16_sums_close(y1, y2, what):
    """Two bf16 outputs of the same fp32 states whose sums over states were formed in two ways
    (terms rounded to bf16 once, 2^-9 relative, then summed in fp32; or summed in fp32): each
    element is then rounded to bf16, so the two may differ by up to two units in the last
    place (2^-6 relative) plus what the terms' rounding leaves after cancellation: up to 2^-9
    of the sum of the terms' magnitudes each way, taken as 2^-6 of the largest output (below
    the 2e-2 of it that both are held to against the oracle)."""
    a, b = y1.double(), y2.double()
    tol = 2 ** -6 * torch.maximum(a.abs(), b.abs()) + 2 ** -6 * b.abs().max()
    bad = (a - b).abs() > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} elements, max |diff| {(a - b).abs().max().item():.3g}"


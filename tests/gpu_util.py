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

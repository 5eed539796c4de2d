"""Pins of the producer-side oracle (delta, B and C from x): values fixed by arithmetic or by
the structure of the inputs, not by re-running the oracle's own formulas.  CPU only."""
import math

import numpy as np
import pytest
import torch

from oracle import producer as P
import workloads


def test_round_bf16_matches_hardware_rne_on_fp32_values():
    # torch's fp32 -> bf16 conversion is round-to-nearest-even; on values exact in fp32 the
    # oracle's direct fp64 rounding must agree bit for bit
    g = np.random.default_rng(1)
    v = np.concatenate([g.standard_normal(20000) * 10.0 ** g.integers(-6, 6, 20000),
                        [1.0, -1.0, 0.0, 3.0e38, 1.17549435e-38]]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    assert np.array_equal(P.round_bf16(v.astype(np.float64)), want)


def test_round_bf16_ties_go_to_even():
    ulp = 2.0 ** -7                                  # bf16 spacing in [1, 2)
    assert P.round_bf16(1.0 + ulp / 2) == 1.0        # tie between 1 and 1+ulp -> even (1)
    assert P.round_bf16(1.0 + 1.5 * ulp) == 1.0 + 2 * ulp
    assert P.round_bf16(1.0 + ulp / 2 + 1e-12) == 1.0 + ulp
    assert P.round_bf16(-(1.0 + ulp / 2)) == -1.0
    assert P.round_bf16(255.5) == 256.0 and P.round_bf16(254.5) == 254.0   # spacing 1 at 128..256... and 2 above
    assert P.round_bf16(257.0) == 256.0 and P.round_bf16(259.0) == 260.0


def test_softplus_closed_forms():
    assert P.softplus(0.0) == pytest.approx(math.log(2.0), rel=1e-15)
    z = np.linspace(-30, 30, 601)
    assert np.allclose(P.softplus(z) - P.softplus(-z), z, rtol=0, atol=1e-12)      # softplus(z) - softplus(-z) = z
    assert np.allclose(P.softplus(np.array([-40.0, -60.0])), np.exp([-40.0, -60.0]), rtol=1e-12)
    assert P.softplus(800.0) == 800.0 and np.isfinite(P.softplus(-800.0))
    assert P.softplus(1.0) == pytest.approx(math.log1p(math.e), rel=1e-15)


def test_rms_norm_hand_values():
    v = np.array([[3.0, 4.0]])                       # mean square 12.5
    out = P.rms_norm(v, [1.0, 2.0], eps=0.0)
    assert np.allclose(out, [[3 / math.sqrt(12.5), 8 / math.sqrt(12.5)]], rtol=1e-15)
    c = np.full((1, 16), -7.25)
    assert np.allclose(P.rms_norm(c, np.ones(16), 0.0), -1.0, rtol=1e-15)      # constant vector -> sign * gain
    assert np.allclose(P.rms_norm(c * 1e-3, np.ones(16), 0.0), -1.0, rtol=1e-15)   # scale invariance
    # eps enters inside the root: v = 0.1 (mean square 0.01), eps = 0.03 -> v / 0.2
    assert np.allclose(P.rms_norm(np.full((1, 4), 0.1), np.ones(4), 0.03), 0.5, rtol=1e-14)


def test_projection_rows_are_outputs_and_split_order():
    """W_x rows select input channels, so before normalisation the outputs are those channels;
    with constant gains the normalised values follow from the selected inputs alone."""
    M, D, R, N = 5, 64, 16, 16
    g = np.random.default_rng(3)
    x = g.standard_normal((M, D))
    sel = g.permutation(D)[:R + 2 * N]
    w_x = np.zeros((R + 2 * N, D))
    w_x[np.arange(R + 2 * N), sel] = 1.0
    w_dt = np.zeros((D, R))
    b_dt = np.zeros(D)
    d_low, B, C, delta = P.ssm_inputs(x, w_x, np.ones(R), np.full(N, 2.0), np.full(N, 0.5), w_dt, b_dt, 0.0, R, N)
    for out, cols, gain in ((d_low, sel[:R], 1.0), (B, sel[R:R + N], 2.0), (C, sel[R + N:], 0.5)):
        v = x[:, cols]
        want = v / np.sqrt((v * v).mean(axis=1, keepdims=True)) * gain
        assert np.array_equal(out, P.round_bf16(want))
    assert np.all(delta == P.round_bf16(math.log(2.0)))    # W_dt = 0, b = 0: softplus(0)


def test_delta_projection_orientation():
    """W_dt rows are output channels: a one-hot W_dt row copies one d_low column."""
    M, D, R = 3, 32, 16
    d_low = P.round_bf16(np.random.default_rng(4).standard_normal((M, R)))
    w_dt = np.zeros((D, R))
    pick = np.arange(D) % R
    w_dt[np.arange(D), pick] = 1.0
    b = np.linspace(-1, 1, D)
    got = P.delta_from_low(d_low, w_dt, b)
    want = P.round_bf16(np.logaddexp(0.0, d_low[:, pick] + b))
    assert np.array_equal(got, want)


def test_producer_weights_give_the_scan_workloads_delta_distribution():
    """Synthetic weights are scaled so delta = softplus(~N(0,1) - 2), mean ~0.18 like the
    scan workloads' directly drawn delta."""
    D, R = 512, 256
    wts = workloads.producer_weights(D, R)
    x = workloads.small_prefill(1, 256, D, "bf16", seed=2)["x"][0].double().numpy()
    _, B, C, delta = P.ssm_inputs(x, wts["w_x"].double().numpy(), wts["g_d"].numpy(), wts["g_b"].numpy(),
                                  wts["g_c"].numpy(), wts["w_dt"].double().numpy(), wts["b_dt"].numpy(), 1e-6, R)
    assert 0.12 < delta.mean() < 0.26 and delta.min() > 0
    assert 0.7 < np.sqrt((B * B).mean()) < 1.3 and 0.7 < np.sqrt((C * C).mean()) < 1.3


# ---- sensitivity: plausible mistakes in the producer oracle each fail a pin ----------------

def _structure_pin(impl):
    """The selection-matrix and one-hot checks above, as a function of an implementation of
    ssm_inputs; returns True when the implementation passes."""
    M, D, R, N = 4, 48, 16, 16
    g = np.random.default_rng(7)
    x = g.standard_normal((M, D))
    sel = g.permutation(D)[:R + 2 * N]
    w_x = np.zeros((R + 2 * N, D))
    w_x[np.arange(R + 2 * N), sel] = 1.0
    w_dt = np.zeros((D, R))
    w_dt[np.arange(D), np.arange(D) % R] = 1.0
    b = np.linspace(-1, 1, D)
    d_low, B, C, delta = impl(x, w_x, np.ones(R), np.full(N, 2.0), np.full(N, 0.5), w_dt, b, 0.0, R, N)
    ok = True
    for out, cols, gain in ((d_low, sel[:R], 1.0), (B, sel[R:R + N], 2.0), (C, sel[R + N:], 0.5)):
        v = x[:, cols]
        ok &= np.array_equal(out, P.round_bf16(v / np.sqrt((v * v).mean(axis=1, keepdims=True)) * gain))
    ok &= np.array_equal(delta, P.round_bf16(np.logaddexp(0.0, d_low[:, np.arange(D) % R] + b)))
    return bool(ok)


def _mutant(kind):
    def impl(x, w_x, g_d, g_b, g_c, w_dt, b_dt, eps, R, N=16):
        x, w_x, w_dt = (np.asarray(a, np.float64) for a in (x, w_x, w_dt))
        proj = x @ w_x.T
        norm = P.rms_norm
        if kind == "sum_not_mean":
            norm = lambda v, g, e: v / np.sqrt((v * v).sum(axis=-1, keepdims=True) + e) * g  # noqa: E731
        d_low = P.round_bf16(norm(proj[:, :R], g_d, eps))
        B = P.round_bf16(norm(proj[:, R:R + N], g_b, eps))
        C = P.round_bf16(norm(proj[:, R + N:], g_c, eps))
        if kind == "swap_bc":
            B, C = C, B
        if kind == "norm_over_all":
            allv = norm(proj, np.ones(R + 2 * N), eps)
            d_low = P.round_bf16(allv[:, :R] * g_d)
        z = d_low @ w_dt.T + b_dt
        if kind == "no_bias":
            z = d_low @ w_dt.T
        if kind == "wdt_transposed":
            z = d_low @ w_dt[:R, :R] + b_dt[:R] if w_dt.shape[0] != R else d_low @ w_dt + b_dt
            z = np.pad(z, ((0, 0), (0, w_dt.shape[0] - z.shape[1])))
        if kind == "no_softplus":
            delta = P.round_bf16(z)
        else:
            delta = P.round_bf16(P.softplus(z))
        return d_low, B, C, delta
    return impl


def test_producer_pin_accepts_the_oracle():
    assert _structure_pin(P.ssm_inputs)


@pytest.mark.parametrize("kind", ["sum_not_mean", "swap_bc", "norm_over_all", "no_bias", "wdt_transposed",
                                  "no_softplus"])
def test_producer_pin_rejects_planted_mistake(kind):
    assert not _structure_pin(_mutant(kind))

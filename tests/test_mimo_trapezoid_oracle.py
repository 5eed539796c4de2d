"""The MIMO scan with the exponential-trapezoidal rule (both Mamba-3 changes together) in the
oracle, pinned to the two pinned oracles it combines, for the diagonal and the complex state:

* lam = 1 is the MIMO scan (oracle.prefill_mimo), whatever the previous token;
* R = 1 is the single-input trapezoidal scan (oracle.prefill_trapezoid);
* superposition over ranks: the recurrence is linear in its inputs (this token's and the
  previous one's) and the decay does not depend on them, so the state is the sum of R
  single-input trapezoidal scans (input r through B's column r, previous token's input r
  through B_prev's column r), and output r' the sum of their read-outs through C's column r';
* a scan resumed from (h, x[L1 - 1], B[L1 - 1]) equals the whole scan.

Planted mistakes in a numpy copy each fail at least one pin (CPU only)."""
import numpy as np
import pytest

import oracle

FORMS = ["diagonal", "complex"]


def _case(seed, form, batch=2, L=25, D=3, N=16, R=4, h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((batch, L, D, R))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    lam = r.uniform(0.0, 1.0, size=(batch, L, D))
    if form == "complex":
        A = np.empty((D, N))
        A[:, 0::2] = -np.arange(1, N // 2 + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N // 2))
        A[:, 1::2] = r.uniform(-np.pi, np.pi, size=(D, N // 2))
    else:
        A = -np.arange(1, N + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N))
    B = r.standard_normal((batch, L, N, R))
    C = r.standard_normal((batch, L, N, R))
    h = r.normal(0.0, 0.5, size=(batch, D, N)) if h0 else None
    xp = r.standard_normal((batch, D, R))
    Bp = r.standard_normal((batch, N, R))
    return x, delta, lam, A, B, C, h, xp, Bp


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def pin_lambda_one_is_mimo(impl):
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(1, form)
        lam[:] = 1.0
        y, h = impl.prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        y_ref, h_ref = oracle.prefill_mimo(x, delta, A, B, C, h0, form)
        assert _rel(y, y_ref) < 1e-13 and _rel(h, h_ref) < 1e-13, f"lam = 1 is not the MIMO scan ({form})"


def pin_rank_one_is_trapezoid(impl):
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(2, form, R=1)
        y, h = impl.prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        y_ref, h_ref = oracle.prefill_trapezoid(x[..., 0], delta, lam, A, B[..., 0], C[..., 0], h0, xp[..., 0],
                                                Bp[..., 0], form)
        assert _rel(y[..., 0], y_ref) < 1e-13 and _rel(h, h_ref) < 1e-13, f"R = 1 is not the trapezoidal scan ({form})"


def pin_superposition(impl):
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(3, form)
        R = x.shape[-1]
        y, h = impl.prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        y_ref = np.zeros_like(y)
        h_ref = 0.0
        for r in range(R):
            start = h0 if r == 0 else None
            for ro in range(R):
                yr, hr = oracle.prefill_trapezoid(x[..., r], delta, lam, A, B[..., r], C[..., ro], start, xp[..., r],
                                                  Bp[..., r], form)
                y_ref[..., ro] += yr
            h_ref = h_ref + hr
        assert _rel(y, y_ref) < 1e-12 and _rel(h, h_ref) < 1e-12, f"not the superposition of trapezoidal scans ({form})"


def pin_resume(impl):
    for form in FORMS:
        x, delta, lam, A, B, C, h0, _, _ = _case(4, form, L=30)
        y, h = impl.prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0, None, None, form)
        L1 = 13
        y1, h1 = impl.prefill_mimo_trapezoid(x[:, :L1], delta[:, :L1], lam[:, :L1], A, B[:, :L1], C[:, :L1], h0, None,
                                             None, form)
        y2, h2 = impl.prefill_mimo_trapezoid(x[:, L1:], delta[:, L1:], lam[:, L1:], A, B[:, L1:], C[:, L1:], h1,
                                             x[:, L1 - 1], B[:, L1 - 1], form)
        assert _rel(np.concatenate([y1, y2], axis=1), y) < 1e-14 and _rel(h2, h) < 1e-14, f"resume ({form})"


PINS = [pin_lambda_one_is_mimo, pin_rank_one_is_trapezoid, pin_superposition, pin_resume]


class _Oracle:
    prefill_mimo_trapezoid = staticmethod(oracle.prefill_mimo_trapezoid)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_Oracle)


def test_step_is_the_one_token_prefill():
    x, delta, lam, A, B, C, h0, xp, Bp = _case(5, "diagonal", L=6)
    y, h = oracle.prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp)
    hs = h0
    for t in range(x.shape[1]):
        xprev, bprev = (xp, Bp) if t == 0 else (x[:, t - 1], B[:, t - 1])
        yt, hs = oracle.step_mimo_trapezoid(hs, xprev, bprev, x[:, t], delta[:, t], lam[:, t], A, B[:, t], C[:, t])
        assert np.array_equal(yt, y[:, t])
    assert np.array_equal(hs, h)


def _numpy_impl(mistake):
    """A numpy copy of the recurrence (both forms, complex arithmetic) with one planted mistake."""

    def prefill_mimo_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form="diagonal"):
        cx = form == "complex"
        pair = (lambda v: v[..., 0::2, :] + 1j * v[..., 1::2, :]) if cx else (lambda v: np.asarray(v, complex))
        batch, L, D, R = x.shape
        a = (A[:, 0::2] + 1j * A[:, 1::2]) if cx else A.astype(complex)
        K = a.shape[1]
        h = np.zeros((batch, D, K), complex)
        if h0 is not None:
            h = (h0[..., 0::2] + 1j * h0[..., 1::2]) if cx else h0.astype(complex)
        u_prev = np.zeros((batch, D, K), complex)
        if x_prev is not None:
            xpv = np.roll(x_prev, 1, axis=-1) if mistake == "previous_ranks_shifted" else x_prev
            u_prev = np.einsum("bkr,bdr->bdk", pair(B_prev), xpv)
        y = np.zeros((batch, L, D, R))
        for t in range(L):
            u = np.einsum("bkr,bdr->bdk", pair(B[:, t]), x[:, t])
            dl, lm = delta[:, t, :, None], lam[:, t, :, None]
            if mistake == "lambda_swapped":
                lm = 1 - lm
            abar = np.exp(dl * a[None])
            left = u if mistake == "left_end_is_this_token" else u_prev
            h = abar * h + (1 - lm) * dl * abar * left + lm * dl * u
            u_prev = u
            y[:, t] = np.real(np.einsum("bkr,bdk->bdr", np.conj(pair(C[:, t])), h))
        if cx:
            out = np.empty((batch, D, 2 * K))
            out[..., 0::2], out[..., 1::2] = h.real, h.imag
        else:
            out = h.real.copy()
        return y, out

    class Impl:
        pass
    Impl.prefill_mimo_trapezoid = staticmethod(prefill_mimo_trapezoid)
    return Impl


def test_faithful_numpy_copy_passes():
    for pin in PINS:
        pin(_numpy_impl(None))


@pytest.mark.parametrize("mistake", ["previous_ranks_shifted", "lambda_swapped", "left_end_is_this_token"])
def test_pins_catch_mistake(mistake):
    failed = []
    for pin in PINS:
        try:
            pin(_numpy_impl(mistake))
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mistake}"

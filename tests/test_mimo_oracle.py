"""The multi-input, multi-output scan (MIMO, the third Mamba-3 change: R inputs and R outputs per
channel, B_t and C_t N x R) in the oracle, against what mathematics fixes, for the diagonal and
the complex-valued state:

* R = 1 is the single-input scan (oracle.prefill / prefill_complex, pinned on their own);
* superposition: the recurrence is linear in its input and the decay does not depend on it,
  so the MIMO state is the sum of R single-input scans (input x[..., r] through B[..., r]),
  and output r' is the sum of those scans read out through C[..., r'];
* brute-force unrolled sums;
* permuting the ranks of x and B together changes nothing; permuting the ranks of C permutes
  the outputs.

Planted mistakes in a numpy copy each fail at least one pin (CPU only)."""
import numpy as np
import pytest

import oracle


def _case(seed, form, batch=2, L=30, D=4, N=16, R=4, h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((batch, L, D, R))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    if form == "complex":
        A = np.empty((D, N))
        A[:, 0::2] = -np.arange(1, N // 2 + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N // 2))
        A[:, 1::2] = r.uniform(-np.pi, np.pi, size=(D, N // 2))
    else:
        A = -np.arange(1, N + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N))
    B = r.standard_normal((batch, L, N, R))
    C = r.standard_normal((batch, L, N, R))
    h = r.normal(0.0, 0.5, size=(batch, D, N)) if h0 else None
    return x, delta, A, B, C, h


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def _siso(form):
    return oracle.prefill_complex if form == "complex" else oracle.prefill


FORMS = ["diagonal", "complex"]


def pin_rank_one(impl):
    for form in FORMS:
        x, delta, A, B, C, h0 = _case(1, form, R=1)
        y, h = impl.prefill_mimo(x, delta, A, B, C, h0, form)
        y_ref, h_ref = _siso(form)(x[..., 0], delta, A, B[..., 0], C[..., 0], h0)
        assert _rel(y[..., 0], y_ref) < 1e-13 and _rel(h, h_ref) < 1e-13, f"R = 1 is not the plain scan ({form})"


def pin_superposition(impl):
    for form in FORMS:
        x, delta, A, B, C, h0 = _case(2, form)
        R = x.shape[-1]
        y, h = impl.prefill_mimo(x, delta, A, B, C, h0, form)
        y_ref = np.zeros_like(y)
        h_ref = 0.0
        for r in range(R):
            start = h0 if r == 0 else None      # the initial state decays once, in one of the parts
            for ro in range(R):
                yr, hr = _siso(form)(x[..., r], delta, A, B[..., r], C[..., ro], start)
                y_ref[..., ro] += yr
            h_ref = h_ref + hr
        assert _rel(y, y_ref) < 1e-12, f"outputs are not the superposition of single-input scans ({form})"
        assert _rel(h, h_ref) < 1e-12, f"state is not the superposition of single-input scans ({form})"


def pin_brute_force(impl):
    """h_t[n] = sum_s (prod_{q=s+1..t} abar_q[n]) delta_s sum_r B_s[n, r] x_s[r] + (prod_{q<=t} abar_q[n]) h0[n]."""
    for form in FORMS:
        x, delta, A, B, C, h0 = _case(3, form, batch=1, L=10, D=2, R=3)
        y, h = impl.prefill_mimo(x, delta, A, B, C, h0, form)
        cx = form == "complex"
        pair = (lambda v: v[..., 0::2, :] + 1j * v[..., 1::2, :]) if cx else (lambda v: v.astype(complex))
        a = (A[:, 0::2] + 1j * A[:, 1::2]) if cx else A.astype(complex)
        hc0 = (h0[0][:, 0::2] + 1j * h0[0][:, 1::2]) if cx else h0[0].astype(complex)
        Bc, Cc = pair(B[0]), pair(C[0])                       # [L, K, R]
        L, D, R = x.shape[1], x.shape[2], x.shape[3]
        for d in range(D):
            for t in range(L):
                ht = np.exp(a[d] * delta[0, :t + 1, d].sum()) * hc0[d]
                for s in range(t + 1):
                    decay = np.exp(a[d] * delta[0, s + 1:t + 1, d].sum())
                    ht = ht + decay * delta[0, s, d] * (Bc[s] * x[0, s, d][None, :]).sum(-1)
                for r in range(R):
                    yt = np.real(np.conj(Cc[t][:, r]) * ht).sum()
                    assert abs(yt - y[0, t, d, r]) <= 1e-12 * max(1.0, abs(yt)), f"brute force y ({form}) t={t}"
            got = (h[0, d, 0::2] + 1j * h[0, d, 1::2]) if cx else h[0, d]
            assert _rel(got, ht) < 1e-12, f"brute force h ({form})"


def pin_rank_permutations(impl):
    for form in FORMS:
        x, delta, A, B, C, h0 = _case(4, form, R=4)
        y, h = impl.prefill_mimo(x, delta, A, B, C, h0, form)
        p = np.array([2, 0, 3, 1])
        y2, h2 = impl.prefill_mimo(x[..., p], delta, A, B[..., p], C, h0, form)
        assert _rel(y2, y) < 1e-13 and _rel(h2, h) < 1e-13, f"joint input-rank permutation changed the scan ({form})"
        y3, h3 = impl.prefill_mimo(x, delta, A, B, C[..., p], h0, form)
        assert np.array_equal(y3, y[..., p]) and np.array_equal(h3, h), f"output ranks not permuted with C ({form})"


PINS = [pin_rank_one, pin_superposition, pin_brute_force, pin_rank_permutations]


class _Oracle:
    prefill_mimo = staticmethod(oracle.prefill_mimo)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_Oracle)


def test_step_chain_equals_prefill():
    for form in FORMS:
        x, delta, A, B, C, h0 = _case(5, form, L=12)
        y, h = oracle.prefill_mimo(x, delta, A, B, C, h0, form)
        hs = h0
        for t in range(x.shape[1]):
            yt, hs = oracle.step_mimo(hs, x[:, t], delta[:, t], A, B[:, t], C[:, t], form)
            assert np.array_equal(yt, y[:, t])
        assert np.array_equal(hs, h)


def test_scalar_form_is_the_expanded_diagonal():
    x, delta, A, B, C, h0 = _case(6, "diagonal")
    a = A[:, 0].copy()
    y, h = oracle.prefill_mimo(x, delta, a, B, C, h0, "scalar")
    y2, h2 = oracle.prefill_mimo(x, delta, np.repeat(a[:, None], 16, 1), B, C, h0, "diagonal")
    assert np.array_equal(y, y2) and np.array_equal(h, h2)


def _numpy_impl(mistake):
    """A numpy copy of the MIMO recurrence (both forms, complex arithmetic) with one planted mistake."""

    def prefill_mimo(x, delta, A, B, C, h0=None, form="diagonal"):
        cx = form == "complex"
        pair = (lambda v: v[..., 0::2, :] + 1j * v[..., 1::2, :]) if cx else (lambda v: np.asarray(v, complex))
        batch, L, D, R = x.shape
        a = (A[:, 0::2] + 1j * A[:, 1::2]) if cx else A.astype(complex)
        K = a.shape[1]
        h = np.zeros((batch, D, K), complex)
        if h0 is not None:
            h = (h0[..., 0::2] + 1j * h0[..., 1::2]) if cx else h0.astype(complex)
        y = np.zeros((batch, L, D, R))
        for t in range(L):
            Bt, Ct = pair(B[:, t]), pair(C[:, t])             # [batch, K, R]
            xt = x[:, t]                                      # [batch, D, R]
            if mistake == "B_layout":                          # the [N][R] rows read as [R][N]
                flat = np.asarray(B[:, t]).reshape(batch, -1)
                Bt = pair(flat.reshape(batch, R, -1).swapaxes(1, 2))
            if mistake == "x_rank_shifted":
                xt = np.roll(xt, 1, axis=-1)
            if mistake == "one_rank_only":
                xt = xt.copy()
                xt[..., 1:] = 0.0
            u = np.einsum("bkr,bdr->bdk", Bt, xt)
            dl = delta[:, t, :, None]
            if mistake == "delta_squared":
                dl = dl * dl
            h = np.exp(dl * a[None]) * h + dl * u
            if mistake == "outputs_summed":
                y[:, t] = np.real(np.einsum("bkr,bdk->bd", np.conj(Ct), h))[..., None]
            elif mistake == "output_uses_B":
                y[:, t] = np.real(np.einsum("bkr,bdk->bdr", np.conj(Bt), h))
            else:
                y[:, t] = np.real(np.einsum("bkr,bdk->bdr", np.conj(Ct), h))
        if cx:
            out = np.empty((batch, D, 2 * K))
            out[..., 0::2], out[..., 1::2] = h.real, h.imag
        else:
            out = h.real.copy()
        return y, out

    class Impl:
        pass
    Impl.prefill_mimo = staticmethod(prefill_mimo)
    return Impl


def test_faithful_numpy_copy_passes():
    impl = _numpy_impl(None)
    for pin in PINS:
        pin(impl)


@pytest.mark.parametrize("mistake", ["B_layout", "x_rank_shifted", "one_rank_only", "delta_squared",
                                     "outputs_summed", "output_uses_B"])
def test_pins_catch_mistake(mistake):
    impl = _numpy_impl(mistake)
    failed = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mistake}"

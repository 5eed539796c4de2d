"""The exponential-trapezoidal rule (the Mamba-3 discretisation) in the oracle, against what
mathematics fixes, for the diagonal and the complex-valued state:

* with lam = 1 it is the Euler rule, i.e. the plain scan (and the complex scan);
* with lam = 1/2 it is the trapezoid rule for the input integral of the continuous system
  h' = a h + b x(s), so its error against the closed-form solution of that ODE falls as the
  square of the step size, on a grid whose steps alternate between two lengths, where the
  Euler rule's falls linearly;
* brute-force unrolled sums, grouped by input token rather than by step;
* a resumed scan (h0 plus the previous token) equals the uninterrupted one, and the decode
  step chain equals the prefill.

Planted mistakes in a numpy copy of the recurrence each fail at least one pin (CPU only)."""
import numpy as np
import pytest

import oracle


def _case(seed, form, batch=2, L=40, D=5, N=16, h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((batch, L, D))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    lam = r.uniform(0.0, 1.0, size=(batch, L, D))
    if form == "complex":
        A = np.empty((D, N))
        A[:, 0::2] = -np.arange(1, N // 2 + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N // 2))
        A[:, 1::2] = r.uniform(-np.pi, np.pi, size=(D, N // 2))
    else:
        A = -np.arange(1, N + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N))
    B = r.standard_normal((batch, L, N))
    C = r.standard_normal((batch, L, N))
    h = r.normal(0.0, 0.5, size=(batch, D, N)) if h0 else None
    xp = r.standard_normal((batch, D))
    Bp = r.standard_normal((batch, N))
    return x, delta, lam, A, B, C, h, xp, Bp


def _cplx(v):
    return v[..., 0::2] + 1j * v[..., 1::2]


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


FORMS = ["diagonal", "complex"]


def pin_euler_reduction(impl):
    """lam = 1: the plain scan (real or complex), whatever the previous token is."""
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(1, form)
        lam[:] = 1.0
        y, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        ref = oracle.prefill_complex if form == "complex" else oracle.prefill
        y_ref, h_ref = ref(x, delta, A, B, C, h0)
        assert _rel(y, y_ref) < 1e-13 and _rel(h, h_ref) < 1e-13, f"lam = 1 is not the Euler rule ({form})"


def _ode_error(impl, form, K, lam_value):
    """Integrate h' = a h + b x(s) over [0, T] on a grid whose steps alternate between lengths
    2/3 s and 4/3 s (s = T / K), x(s) = cos(w s + phi), constant b, and return the largest
    error of the final state against the ODE's closed-form solution."""
    T, w = 2.0, 3.0
    D = 3
    phi = np.array([0.1, 0.9, 2.0])
    r = np.random.default_rng(7)
    if form == "complex":
        N = 8
        A = np.empty((D, N))
        A[:, 0::2] = -r.uniform(0.3, 2.0, size=(D, N // 2))
        A[:, 1::2] = r.uniform(-4.0, 4.0, size=(D, N // 2))
        a = _cplx(A)
    else:
        N = 4
        A = -r.uniform(0.3, 2.0, size=(D, N))
        a = A.astype(complex)
    bv = r.standard_normal(N)
    b = _cplx(bv) if form == "complex" else bv.astype(complex)
    steps = np.where(np.arange(K) % 2 == 0, 2.0 / 3.0, 4.0 / 3.0) * (T / K)
    grid = np.concatenate([[0.0], np.cumsum(steps)])        # grid[K] == T
    xs = np.cos(w * grid[:, None] + phi[None, :])            # [K + 1, D]
    h0 = r.normal(0, 1, size=(1, D, N))
    x = xs[1:][None]
    delta = np.broadcast_to(steps[:, None], (K, D))[None].copy()
    lam = np.full_like(x, lam_value)
    B = np.broadcast_to(bv, (1, K, N)).copy()
    C = np.broadcast_to(np.ones(N), (1, K, N)).copy()
    _, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, h0, xs[0][None], bv[None], form)
    # closed form: h(T) = e^{aT} h(0) + b e^{aT} Re-or-complex[ e^{i phi} (e^{(iw - a)T} - 1) / (iw - a) ] for cos
    hT0 = _cplx(h0[0]) if form == "complex" else h0[0].astype(complex)
    aa = a[:, :, None]                                       # [D, K', 1]
    ip, im = np.exp(1j * phi)[:, None, None], np.exp(-1j * phi)[:, None, None]
    # cos = (e^{i.} + e^{-i.}) / 2, each term integrated exactly
    integ = 0.5 * (ip * (np.exp((1j * w - aa) * T) - 1) / (1j * w - aa)
                   + im * (np.exp((-1j * w - aa) * T) - 1) / (-1j * w - aa))[..., 0]
    exact = np.exp(a * T) * hT0 + b[None] * np.exp(a * T) * integ
    got = _cplx(h[0]) if form == "complex" else h[0]
    return float(np.max(np.abs(got - exact)))


def pin_second_order(impl):
    """lam = 1/2 converges as the square of the step size (on alternating step lengths); lam = 1
    (the Euler rule) only linearly.  Both forms."""
    for form in FORMS:
        e1, e2, e3 = (_ode_error(impl, form, K, 0.5) for K in (200, 400, 800))
        assert 3.6 < e1 / e2 < 4.4 and 3.6 < e2 / e3 < 4.4, f"trapezoid not second order ({form}: {e1}, {e2}, {e3})"
        f1, f2 = (_ode_error(impl, form, K, 1.0) for K in (400, 800))
        assert 1.8 < f1 / f2 < 2.2, f"Euler not first order ({form}: {f1}, {f2})"
        assert e2 < f1 / 20, "trapezoid no better than Euler"


def pin_brute_force(impl):
    """Unrolled by input token: u_s = B_s x_s enters h_t with weight
    prod_{r=s+1..t} abar_r * (lam_s delta_s + (1 - lam_{s+1}) delta_{s+1} [s < t]), the token
    before the first (s = -1) with (1 - lam_0) delta_0 prod_{r=0..t} abar_r."""
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(5, form, 1, 12, 3)
        y, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        cx = form == "complex"
        a = _cplx(A) if cx else A.astype(complex)
        Bc = _cplx(B[0]) if cx else B[0].astype(complex)
        Cc = _cplx(C[0]) if cx else C[0].astype(complex)
        Bpc = _cplx(Bp[0]) if cx else Bp[0].astype(complex)
        h0c = _cplx(h0[0]) if cx else h0[0].astype(complex)
        L, D = x.shape[1], x.shape[2]
        for d in range(D):
            abar = [np.exp(delta[0, t, d] * a[d]) for t in range(L)]

            def prod(lo, hi):            # prod_{r=lo..hi} abar_r
                p = np.ones_like(a[d])
                for rr in range(lo, hi + 1):
                    p = p * abar[rr]
                return p
            for t in range(L):
                ht = prod(0, t) * h0c[d] + (1 - lam[0, 0, d]) * delta[0, 0, d] * prod(0, t) * Bpc * xp[0, d]
                for s in range(t + 1):
                    wgt = lam[0, s, d] * delta[0, s, d]
                    if s < t:
                        wgt = wgt + (1 - lam[0, s + 1, d]) * delta[0, s + 1, d]
                    ht = ht + prod(s + 1, t) * wgt * Bc[s] * x[0, s, d]
                yt = np.real(np.conj(Cc[t]) * ht).sum()
                assert abs(yt - y[0, t, d]) <= 1e-12 * max(1.0, abs(yt)), f"brute force y ({form}) t={t} d={d}"
            got = _cplx(h[0, d]) if cx else h[0, d]
            assert _rel(got, ht) < 1e-12, f"brute force h ({form})"


def pin_resume(impl):
    """A scan cut after L1 tokens and resumed from (h, x[L1 - 1], B[L1 - 1]) is the whole scan."""
    for form in FORMS:
        x, delta, lam, A, B, C, h0, _, _ = _case(6, form, 2, 30, 4)
        y, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, h0, None, None, form)
        L1 = 11
        y1, h1 = impl.prefill_trapezoid(x[:, :L1], delta[:, :L1], lam[:, :L1], A, B[:, :L1], C[:, :L1], h0, None,
                                        None, form)
        y2, h2 = impl.prefill_trapezoid(x[:, L1:], delta[:, L1:], lam[:, L1:], A, B[:, L1:], C[:, L1:], h1,
                                        x[:, L1 - 1], B[:, L1 - 1], form)
        assert _rel(np.concatenate([y1, y2], axis=1), y) < 1e-14 and _rel(h2, h) < 1e-14, f"resume ({form})"


def pin_first_token_has_no_left_end(impl):
    """Without a previous token the first step takes only lam_0 delta_0 B_0 x_0.  With x zero
    from token 1 on, u_0 = B_0 x_0 is the only input: it enters at token 0 (weight lam_0 delta_0)
    and again as token 1's left end (weight (1 - lam_1) delta_1, decayed over step 1), then
    decays, so from a zero state h_{L-1} = u_0 (lam_0 delta_0 + (1 - lam_1) delta_1)
    exp(A (delta_1 + ... + delta_{L-1}))."""
    x, delta, lam, A, B, C, _, _, _ = _case(8, "diagonal", 1, 6, 2, h0=False)
    x[:, 1:] = 0.0
    y, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, None, None, None, "diagonal")
    S = delta[0, 1:].sum(axis=0)                             # [D]
    wgt = lam[0, 0] * delta[0, 0] + (1 - lam[0, 1]) * delta[0, 1]
    expect = (wgt * x[0, 0])[:, None] * B[0, 0][None, :] * np.exp(S[:, None] * A)
    assert _rel(h[0], expect) < 1e-13, "first token"


def pin_prefill_equals_steps(impl):
    for form in FORMS:
        x, delta, lam, A, B, C, h0, xp, Bp = _case(9, form, 2, 25, 4)
        y, h = impl.prefill_trapezoid(x, delta, lam, A, B, C, h0, xp, Bp, form)
        hs = h0.copy()
        for t in range(x.shape[1]):
            xprev, bprev = (xp, Bp) if t == 0 else (x[:, t - 1], B[:, t - 1])
            yt, hs = impl.step_trapezoid(hs, xprev, bprev, x[:, t], delta[:, t], lam[:, t], A, B[:, t], C[:, t], form)
            assert np.array_equal(yt, y[:, t]), f"step y differs at {t} ({form})"
        assert np.array_equal(hs, h), f"step chain differs from the prefill ({form})"


PINS = [pin_euler_reduction, pin_second_order, pin_brute_force, pin_resume, pin_first_token_has_no_left_end,
        pin_prefill_equals_steps]


class _Oracle:
    prefill_trapezoid = staticmethod(oracle.prefill_trapezoid)
    step_trapezoid = staticmethod(oracle.step_trapezoid)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_Oracle)


def test_scalar_form_is_the_expanded_diagonal():
    x, delta, lam, A, B, C, h0, xp, Bp = _case(10, "diagonal", 1, 20, 6)
    a = A[:, 0].copy()
    y, h = oracle.prefill_trapezoid(x, delta, lam, a, B, C, h0, xp, Bp, "scalar")
    y2, h2 = oracle.prefill_trapezoid(x, delta, lam, np.repeat(a[:, None], 16, 1), B, C, h0, xp, Bp, "diagonal")
    assert np.array_equal(y, y2) and np.array_equal(h, h2)


def _numpy_impl(mistake):
    """A numpy copy of the trapezoid recurrence (both forms, in complex arithmetic) with one
    planted mistake."""

    def prefill_trapezoid(x, delta, lam, A, B, C, h0=None, x_prev=None, B_prev=None, form="diagonal"):
        cx = form == "complex"
        conv = _cplx if cx else (lambda v: np.asarray(v, float).astype(complex))
        batch, L, D = x.shape
        a = conv(A)
        K = a.shape[1]
        h = np.zeros((batch, D, K), complex) if h0 is None else conv(h0).copy()
        u_prev = np.zeros((batch, D, K), complex)
        if x_prev is not None and mistake != "x_prev_ignored":
            u_prev = conv(B_prev)[:, None, :] * np.asarray(x_prev)[:, :, None]
        y = np.zeros((batch, L, D))
        for t in range(L):
            dl = delta[:, t, :, None]
            lm = lam[:, t, :, None]
            if mistake == "lambda_swapped":
                lm = 1 - lm
            u_t = conv(B[:, t])[:, None, :] * x[:, t, :, None]
            abar = np.exp(dl * a[None])
            d_left = dl
            if mistake == "previous_delta" and t > 0:
                d_left = delta[:, t - 1, :, None]
            if mistake == "left_undecayed":
                h = abar * h + (1 - lm) * d_left * u_prev + lm * dl * u_t
            elif mistake == "decay_on_right":
                h = abar * h + (1 - lm) * d_left * u_prev + lm * dl * abar * u_t
            else:
                h = abar * h + (1 - lm) * d_left * abar * u_prev + lm * dl * u_t
            if mistake == "current_B_on_left" and t + 1 < L:
                u_prev = conv(B[:, t + 1])[:, None, :] * x[:, t, :, None]
            else:
                u_prev = u_t
            y[:, t] = np.real(np.conj(conv(C[:, t]))[:, None, :] * h).sum(-1)
        if cx:
            out = np.empty((batch, D, 2 * K))
            out[..., 0::2], out[..., 1::2] = h.real, h.imag
        else:
            out = h.real.copy()
        return y, out

    class Impl:
        pass
    Impl.prefill_trapezoid = staticmethod(prefill_trapezoid)
    return Impl


def test_faithful_numpy_copy_passes():
    impl = _numpy_impl(None)
    for pin in PINS[:-1]:
        pin(impl)


@pytest.mark.parametrize("mistake", ["lambda_swapped", "left_undecayed", "decay_on_right", "previous_delta",
                                     "current_B_on_left", "x_prev_ignored"])
def test_pins_catch_mistake(mistake):
    impl = _numpy_impl(mistake)
    failed = []
    for pin in PINS[:-1]:
        try:
            pin(impl)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mistake}"

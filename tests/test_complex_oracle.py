"""The complex-valued state (the Mamba-3 change; pairs of the N real state components read as
N/2 complex states) in the oracle, against what mathematics fixes: the reduction to the real
scan when A has no imaginary part, a pure rotation that keeps |h|, the closed-form geometric
series with a complex ratio, and brute-force unrolled sums.  Planted mistakes in a numpy copy
of the recurrence each fail at least one pin (CPU only)."""
import numpy as np
import pytest

import oracle


def _case(seed, batch=2, L=40, D=5, N=16, h0=True):
    r = np.random.default_rng(seed)
    x = r.standard_normal((batch, L, D))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    A = np.empty((D, N))
    A[:, 0::2] = -np.arange(1, N // 2 + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N // 2))
    A[:, 1::2] = r.uniform(-np.pi, np.pi, size=(D, N // 2))
    B = r.standard_normal((batch, L, N))
    C = r.standard_normal((batch, L, N))
    h = r.normal(0.0, 0.5, size=(batch, D, N)) if h0 else None
    return x, delta, A, B, C, h


def _cplx(v):
    return v[..., 0::2] + 1j * v[..., 1::2]


def _rel(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / max(np.max(np.abs(b)), 1e-300))


def pin_real_reduction(impl):
    """Imaginary parts zero: the real diagonal scan with A[2k + 1] = A[2k]."""
    x, delta, A, B, C, h0 = _case(1)
    A[:, 1::2] = 0.0
    y, h = impl.prefill_complex(x, delta, A, B, C, h0)
    Ar = A.copy()
    Ar[:, 1::2] = A[:, 0::2]
    y_ref, h_ref = oracle.prefill(x, delta, Ar, B, C, h0)
    assert _rel(y, y_ref) < 1e-13 and _rel(h, h_ref) < 1e-13, "no rotation: not the real scan"


def pin_pure_rotation(impl):
    """Real parts zero and B = 0: each complex state turns by theta_k * sum(delta) and keeps its
    modulus."""
    x, delta, A, B, C, h0 = _case(2)
    A[:, 0::2] = 0.0
    B[:] = 0.0
    y, h = impl.prefill_complex(x, delta, A, B, C, h0)
    S = delta.sum(axis=1)                                      # [b, D]
    theta = A[:, 1::2]                                         # [D, K]
    expect = _cplx(h0) * np.exp(1j * S[:, :, None] * theta[None])
    assert _rel(_cplx(h), expect) < 1e-12, "rotation angle or direction wrong"
    assert np.allclose(np.abs(_cplx(h)), np.abs(_cplx(h0)), rtol=1e-12), "rotation changed the modulus"
    # y_t from the rotated initial state alone
    St = np.cumsum(delta, axis=1)                              # [b, L, D]
    ht = _cplx(h0)[:, None] * np.exp(1j * St[..., None] * theta[None, None])
    y_ref = np.real(np.conj(_cplx(C))[:, :, None, :] * ht).sum(-1)
    assert _rel(y, y_ref) < 1e-12, "output of a rotating state wrong"


def pin_geometric(impl):
    """Constant delta, x and B: h_t = a^(t+1) h0 + b (1 - a^(t+1)) / (1 - a) with complex a."""
    r = np.random.default_rng(3)
    L, D, N = 200, 3, 16
    dl = np.array([0.05, 0.4, 1.5])
    xv = np.array([1.0, -0.7, 0.3])
    _, _, A, _, _, _ = _case(4, 1, 1, D, N, False)
    Bv = r.standard_normal(N)
    Cv = r.standard_normal(N)
    h0 = r.normal(0, 1, size=(1, D, N))
    x = np.broadcast_to(xv, (1, L, D)).copy()
    delta = np.broadcast_to(dl, (1, L, D)).copy()
    B = np.broadcast_to(Bv, (1, L, N)).copy()
    C = np.broadcast_to(Cv, (1, L, N)).copy()
    y, h = impl.prefill_complex(x, delta, A, B, C, h0)
    a = np.exp(dl[:, None] * _cplx(A))                         # [D, K]
    b = (dl * xv)[:, None] * _cplx(Bv)[None, :]
    t = np.arange(L)[:, None, None]
    p = a[None] ** (t + 1)
    ht = p * _cplx(h0[0])[None] + b[None] * (1 - p) / (1 - a[None])
    y_ref = np.real(np.conj(_cplx(Cv))[None, None, :] * ht).sum(-1)[None]
    assert _rel(y, y_ref) < 1e-11, f"geometric y {_rel(y, y_ref)}"
    assert _rel(_cplx(h[0]), ht[-1]) < 1e-11, "geometric h"


def pin_brute_force(impl):
    """Unrolled sums: h_t = sum_s (prod_{r=s+1..t} abar_r) delta_s x_s b_s + (prod_{r<=t} abar_r) h0."""
    x, delta, A, B, C, h0 = _case(5, 1, 14, 3)
    y, h = impl.prefill_complex(x, delta, A, B, C, h0)
    a = _cplx(A)
    L, D = x.shape[1], x.shape[2]
    for d in range(D):
        for t in range(L):
            acc = np.zeros(8, complex)
            for s in range(t + 1):
                prod = np.ones(8, complex)
                for rr in range(s + 1, t + 1):
                    prod = prod * np.exp(delta[0, rr, d] * a[d])
                acc += prod * delta[0, s, d] * x[0, s, d] * _cplx(B[0, s])
            prod = np.ones(8, complex)
            for rr in range(t + 1):
                prod = prod * np.exp(delta[0, rr, d] * a[d])
            ht = acc + prod * _cplx(h0[0, d])
            yt = np.real(np.conj(_cplx(C[0, t])) * ht).sum()
            assert abs(yt - y[0, t, d]) <= 1e-12 * max(1.0, abs(yt)), f"brute force y at t={t} d={d}"
        assert _rel(_cplx(h[0, d]), ht) < 1e-12, "brute force h"


def pin_prefill_equals_steps(impl):
    x, delta, A, B, C, h0 = _case(6, 2, 25, 4)
    y, h = impl.prefill_complex(x, delta, A, B, C, h0)
    hs = h0.copy()
    for t in range(x.shape[1]):
        yt, hs = impl.step_complex(hs, x[:, t], delta[:, t], A, B[:, t], C[:, t])
        assert np.array_equal(yt, y[:, t]), f"step y differs at {t}"
    assert np.array_equal(hs, h), "step chain differs from the prefill"


PINS = [pin_real_reduction, pin_pure_rotation, pin_geometric, pin_brute_force, pin_prefill_equals_steps]


class _Oracle:
    prefill_complex = staticmethod(oracle.prefill_complex)
    step_complex = staticmethod(oracle.step_complex)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_Oracle)


def _numpy_impl(mistake):
    """A numpy copy of the complex recurrence with one planted mistake."""

    def prefill_complex(x, delta, A, B, C, h0=None):
        batch, L, D = x.shape
        a = _cplx(A)
        if mistake == "conjugate_rotation":
            a = np.conj(a)
        h = np.zeros((batch, D, 8), complex) if h0 is None else _cplx(np.asarray(h0, float)).copy()
        y = np.zeros((batch, L, D))
        for t in range(L):
            dl = delta[:, t, :, None]
            bt = _cplx(B[:, t])[:, None, :]
            if mistake == "swapped_B_pair":
                bt = np.conj(bt) * 1j
            ct = _cplx(C[:, t])[:, None, :]
            abar = np.exp(dl * a[None])
            if mistake == "rotation_dropped":
                abar = np.abs(abar)
            h = abar * h + dl * x[:, t, :, None] * bt
            if mistake == "imaginary_output":
                y[:, t] = np.imag(np.conj(ct) * h).sum(-1)
            elif mistake == "unconjugated_C":
                y[:, t] = np.real(ct * h).sum(-1)
            else:
                y[:, t] = np.real(np.conj(ct) * h).sum(-1)
        out = np.empty((batch, D, 16))
        out[..., 0::2], out[..., 1::2] = h.real, h.imag
        return y, out

    class Impl:
        pass
    Impl.prefill_complex = staticmethod(prefill_complex)
    return Impl


def test_faithful_numpy_copy_passes():
    impl = _numpy_impl(None)
    for pin in PINS[:-1]:
        pin(impl)


@pytest.mark.parametrize("mistake", ["conjugate_rotation", "swapped_B_pair", "rotation_dropped", "imaginary_output",
                                     "unconjugated_C"])
def test_pins_catch_mistake(mistake):
    impl = _numpy_impl(mistake)
    failed = 0
    for pin in PINS[:-1]:
        try:
            pin(impl)
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin caught {mistake}"

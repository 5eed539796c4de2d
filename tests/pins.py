"""Pins for a selective-scan implementation, each fixed by mathematics rather than by
re-running the implementation's own formula.

Every pin takes an ``impl`` object with ``prefill(x, delta, A, B, C, h0=None) -> (y, h)``
and ``step(h, x_t, delta_t, A, B_t, C_t) -> (y_t, h_new)`` (float64 numpy in and out)
and raises ``AssertionError`` when the implementation misses.  The test suite runs them
against the oracle (which must pass every one) and against deliberately broken variants
(each of which must fail at least one).

The scan pinned here is the S6 recurrence of the Jamba notes page (section "Mamba layer"):
h_t = exp(Delta_t A) h_{t-1} + Delta_t B_t x_t, y_t = C_t h_t, with diagonal A.
"""
from __future__ import annotations

import math

import numpy as np

try:
    import mpmath
except ImportError:  # pragma: no cover - mpmath ships with the image
    mpmath = None


def _rng(seed):
    return np.random.default_rng(seed)


def random_case(seed, batch=1, L=24, D=3, N=16, h0=True):
    """Small random inputs with the workloads' distributions (delta > 0, A < 0)."""
    r = _rng(seed)
    x = r.standard_normal((batch, L, D))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    A = -np.arange(1, N + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N))
    B = r.standard_normal((batch, L, N))
    C = r.standard_normal((batch, L, N))
    h = r.normal(0.0, 0.5, size=(batch, D, N)) if h0 else None
    return x, delta, A, B, C, h


def _rel(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))) / scale)


# --------------------------------------------------------------------------------------
# P1: brute-force unrolled sums.  The state after token t is the sum over every earlier
# token s of its input term Delta_s B_s x_s carried forward by the product of the decays
# of the tokens after it, plus the initial state carried by all decays.
# --------------------------------------------------------------------------------------
def brute_force_f64(x, delta, A, B, C, h0):
    batch, L, D = x.shape
    N = A.shape[1]
    y = np.zeros((batch, L, D))
    hT = np.zeros((batch, D, N))
    for b in range(batch):
        for d in range(D):
            for n in range(N):
                decay = np.exp(delta[b, :, d] * A[d, n])  # Abar_r for every token r
                for t in range(L):
                    total = 0.0
                    for s in range(t + 1):
                        carry = 1.0
                        for r in range(s + 1, t + 1):
                            carry *= decay[r]
                        total += carry * delta[b, s, d] * B[b, s, n] * x[b, s, d]
                    carry0 = 1.0
                    for r in range(t + 1):
                        carry0 *= decay[r]
                    h_t = total + carry0 * (0.0 if h0 is None else h0[b, d, n])
                    y[b, t, d] += C[b, t, n] * h_t
                    if t == L - 1:
                        hT[b, d, n] = h_t
    return y, hT


def pin_brute_force(impl, seed=1):
    for h0flag, (batch, L, D, N) in [(False, (1, 12, 3, 16)), (True, (2, 9, 2, 5))]:
        x, delta, A, B, C, h0 = random_case(seed, batch, L, D, N, h0flag)
        y, h = impl.prefill(x, delta, A, B, C, h0)
        y_ref, h_ref = brute_force_f64(x, delta, A, B, C, h0)
        assert _rel(y, y_ref) < 1e-13, f"brute force y mismatch {_rel(y, y_ref)}"
        assert _rel(h, h_ref) < 1e-13, f"brute force h mismatch {_rel(h, h_ref)}"


def pin_mpmath(impl, seed=2):
    """Exact (50-digit) unrolled sums on a tiny case; decays taken as exp(A * sum of deltas)."""
    if mpmath is None:
        return
    mpmath.mp.dps = 50
    x, delta, A, B, C, h0 = random_case(seed, 1, 6, 2, 4, True)
    y, h = impl.prefill(x, delta, A, B, C, h0)
    L, D, N = 6, 2, 4
    mp = mpmath.mpf
    for d in range(D):
        for t in range(L):
            yt = mp(0)
            for n in range(N):
                acc = mp(0)
                for s in range(t + 1):
                    tail = sum((mp(delta[0, r, d]) for r in range(s + 1, t + 1)), mp(0))
                    acc += mpmath.exp(mp(A[d, n]) * tail) * mp(delta[0, s, d]) * mp(B[0, s, n]) * mp(x[0, s, d])
                head = sum((mp(delta[0, r, d]) for r in range(t + 1)), mp(0))
                ht = acc + mpmath.exp(mp(A[d, n]) * head) * mp(h0[0, d, n])
                yt += mp(C[0, t, n]) * ht
                if t == L - 1:
                    assert abs(float(ht) - h[0, d, n]) <= 1e-14 * max(1.0, abs(float(ht))), "mpmath h mismatch"
            assert abs(float(yt) - y[0, t, d]) <= 1e-14 * max(1.0, float(mpmath.fabs(yt))) * N, "mpmath y mismatch"


# --------------------------------------------------------------------------------------
# P2: closed-form geometric series.  With Delta, B, C and x constant in time the decay
# abar = exp(Delta A) and the input term b = Delta B x are constant, so
#   h_t = abar^(t+1) h0 + b (1 - abar^(t+1)) / (1 - abar)   ->  b / (1 - abar).
# --------------------------------------------------------------------------------------
def pin_geometric(impl, seed=3):
    r = _rng(seed)
    L, D, N = 300, 4, 16
    dl = np.array([0.05, 0.3, 1.0, 2.5])              # one constant delta per channel
    xv = np.array([1.0, -0.5, 2.0, 0.25])
    A = -np.arange(1, N + 1)[None, :] * r.uniform(0.5, 1.5, size=(D, N))
    Bv = r.standard_normal(N)
    Cv = r.standard_normal(N)
    h0 = r.normal(0, 1, size=(1, D, N))
    x = np.broadcast_to(xv, (1, L, D)).copy()
    delta = np.broadcast_to(dl, (1, L, D)).copy()
    B = np.broadcast_to(Bv, (1, L, N)).copy()
    C = np.broadcast_to(Cv, (1, L, N)).copy()
    y, h = impl.prefill(x, delta, A, B, C, h0)
    abar = np.exp(dl[:, None] * A)                      # [D, N]
    b = dl[:, None] * Bv[None, :] * xv[:, None]         # [D, N]
    t = np.arange(L)[:, None, None]
    p = abar[None] ** (t + 1)
    h_t = p * h0[0][None] + b[None] * (1 - p) / (1 - abar[None])
    y_ref = np.einsum("n,tdn->td", Cv, h_t)[None]
    assert _rel(y, y_ref) < 1e-12, f"geometric y mismatch {_rel(y, y_ref)}"
    assert _rel(h, h_t[-1][None]) < 1e-12, "geometric h mismatch"
    # the fixed point b / (1 - abar) is reached for the fast-decaying channels
    fixed = b / (1 - abar)
    assert np.allclose(h[0, 2:], fixed[2:], rtol=1e-12, atol=1e-12), "fixed point not reached"


# --------------------------------------------------------------------------------------
# P3: chunked evaluation through the associative combine equals the sequential scan.
# --------------------------------------------------------------------------------------
def pin_chunked(impl, seed=4):
    if not hasattr(impl, "prefill_chunked"):
        return
    x, delta, A, B, C, h0 = random_case(seed, 2, 130, 5, 16, True)
    y, h = impl.prefill(x, delta, A, B, C, h0)
    for k in (1, 7, 64, 130, 500):
        yk, hk = impl.prefill_chunked(x, delta, A, B, C, k, h0)
        assert _rel(yk, y) < 1e-12, f"chunk {k}: y differs {_rel(yk, y)}"
        assert _rel(hk, h) < 1e-12, f"chunk {k}: h differs"


# --------------------------------------------------------------------------------------
# P4: prefill equals L successive decode steps (same arithmetic, so bit-identical).
# --------------------------------------------------------------------------------------
def pin_prefill_equals_steps(impl, seed=5):
    x, delta, A, B, C, h0 = random_case(seed, 2, 40, 6, 16, True)
    y, h = impl.prefill(x, delta, A, B, C, h0)
    hs = h0.copy()
    for t in range(x.shape[1]):
        yt, hs = impl.step(hs, x[:, t], delta[:, t], A, B[:, t], C[:, t])
        assert np.array_equal(yt, y[:, t]), f"step y differs at token {t}"
    assert np.array_equal(hs, h), "step chain final state differs from prefill"


# --------------------------------------------------------------------------------------
# P5: A = 0 reduces the scan to a prefix sum.  abar = exp(0) = 1 and with Delta = 0.5,
# B = 2, x = 1, C = 1 every input term is exactly 1, so h_t = t + 1 and y_t = N (t + 1).
# --------------------------------------------------------------------------------------
def pin_prefix_sum(impl):
    L, D, N = 200, 3, 16
    x = np.ones((1, L, D))
    delta = np.full((1, L, D), 0.5)
    A = np.zeros((D, N))
    B = np.full((1, L, N), 2.0)
    C = np.ones((1, L, N))
    y, h = impl.prefill(x, delta, A, B, C, None)
    expect = np.cumsum(np.ones(L))
    assert np.array_equal(y[0, :, 0], N * expect), "A=0 prefix sum y wrong"
    assert np.array_equal(h[0], np.full((D, N), float(L))), "A=0 prefix sum h wrong"
    # with a varying input the A=0 state is the cumulative sum of the input terms
    r = _rng(6)
    x2 = r.standard_normal((1, L, D))
    d2 = np.logaddexp(0, r.standard_normal((1, L, D)) - 2)
    B2 = r.standard_normal((1, L, N))
    y2, h2 = impl.prefill(x2, d2, A, B2, C, None)
    csum = np.cumsum(d2[0, :, :, None] * B2[0, :, None, :] * x2[0, :, :, None], axis=0)  # [L, D, N]
    assert _rel(h2[0], csum[-1]) < 1e-12, "A=0 cumulative sum h wrong"
    assert _rel(y2[0], csum.sum(axis=2)) < 1e-12, "A=0 cumulative sum y wrong"


# --------------------------------------------------------------------------------------
# P6: B = 0 (or x = 0) leaves only the decay path: h_t = exp(A * sum_{s<=t} Delta_s) h0.
# --------------------------------------------------------------------------------------
def pin_decay_only(impl, seed=7):
    x, delta, A, B, C, h0 = random_case(seed, 1, 64, 4, 16, True)
    for zero in ("B", "x"):
        Bz = np.zeros_like(B) if zero == "B" else B
        xz = np.zeros_like(x) if zero == "x" else x
        y, h = impl.prefill(xz, delta, A, Bz, C, h0)
        cums = np.cumsum(delta[0], axis=0)                       # [L, D]
        h_t = np.exp(cums[:, :, None] * A[None]) * h0[0][None]  # [L, D, N]
        assert _rel(h[0], h_t[-1]) < 1e-13, f"decay-only h wrong ({zero}=0)"
        assert _rel(y[0], np.einsum("tn,tdn->td", C[0], h_t)) < 1e-13, f"decay-only y wrong ({zero}=0)"


# --------------------------------------------------------------------------------------
# P7: linearity in the input path.  Doubling x or B doubles every input term exactly;
# negating x negates it; doubling C doubles y only.  With h0 = 0 all of these are exact.
# --------------------------------------------------------------------------------------
def pin_scaling(impl, seed=8):
    x, delta, A, B, C, _ = random_case(seed, 1, 50, 4, 16, False)
    y, h = impl.prefill(x, delta, A, B, C, None)
    y2, h2 = impl.prefill(2 * x, delta, A, B, C, None)
    assert np.array_equal(y2, 2 * y) and np.array_equal(h2, 2 * h), "y(2x) != 2 y(x)"
    yb, hb = impl.prefill(x, delta, A, 2 * B, C, None)
    assert np.array_equal(yb, 2 * y) and np.array_equal(hb, 2 * h), "y(2B) != 2 y(B)"
    yn, hn = impl.prefill(-x, delta, A, B, C, None)
    assert np.array_equal(yn, -y) and np.array_equal(hn, -h), "y(-x) != -y(x)"
    yc, hc = impl.prefill(x, delta, A, B, 2 * C, None)
    assert np.array_equal(yc, 2 * y) and np.array_equal(hc, h), "doubling C must double y only"


# --------------------------------------------------------------------------------------
# P8: causality.  Changing tokens after t0 cannot change any output up to t0.
# --------------------------------------------------------------------------------------
def pin_causality(impl, seed=9):
    x, delta, A, B, C, h0 = random_case(seed, 1, 60, 4, 16, True)
    y, _ = impl.prefill(x, delta, A, B, C, h0)
    t0 = 25
    r = _rng(seed + 100)
    x2, d2, B2, C2 = x.copy(), delta.copy(), B.copy(), C.copy()
    x2[:, t0 + 1:] = r.standard_normal(x2[:, t0 + 1:].shape)
    d2[:, t0 + 1:] = 3.0
    B2[:, t0 + 1:] *= -1
    C2[:, t0 + 1:] += 1
    yp, _ = impl.prefill(x2, d2, A, B2, C2, h0)
    assert np.array_equal(yp[:, :t0 + 1], y[:, :t0 + 1]), "output depends on future tokens"
    assert not np.array_equal(yp[:, t0 + 1:], y[:, t0 + 1:]), "output ignores its own token"


# --------------------------------------------------------------------------------------
# P9: channels are independent.  Permuting channels (x, delta, A rows and h0 together)
# permutes y and the state the same way.
# --------------------------------------------------------------------------------------
def pin_channel_permutation(impl, seed=10):
    x, delta, A, B, C, h0 = random_case(seed, 2, 30, 7, 16, True)
    y, h = impl.prefill(x, delta, A, B, C, h0)
    perm = _rng(seed).permutation(7)
    yp, hp = impl.prefill(x[:, :, perm], delta[:, :, perm], A[perm], B, C, h0[:, perm])
    assert np.array_equal(yp, y[:, :, perm]) and np.array_equal(hp, h[:, perm]), "channel permutation broke"
    # the two batch rows are independent too
    y1, h1 = impl.prefill(x[1:], delta[1:], A, B[1:], C[1:], h0[1:])
    assert np.array_equal(y1, y[1:]) and np.array_equal(h1, h[1:]), "batch rows interact"


# --------------------------------------------------------------------------------------
# P10: Delta = 0 freezes the state: abar = 1, input term 0, y_t = C_t h0.
# --------------------------------------------------------------------------------------
def pin_zero_delta(impl, seed=11):
    x, delta, A, B, C, h0 = random_case(seed, 1, 20, 3, 16, True)
    y, h = impl.prefill(x, np.zeros_like(delta), A, B, C, h0)
    assert np.array_equal(h, h0), "delta = 0 must keep the state"
    y_ref = np.einsum("tn,dn->td", C[0], h0[0])
    assert _rel(y[0], y_ref) < 1e-14, "delta = 0 output wrong"


# --------------------------------------------------------------------------------------
# P11: state size is [batch, D, N], independent of L (notes page, "KV cache efficiency").
# --------------------------------------------------------------------------------------
def pin_state_shape(impl, seed=12):
    for L in (1, 17, 64):
        x, delta, A, B, C, _ = random_case(seed, 2, L, 3, 16, False)
        y, h = impl.prefill(x, delta, A, B, C, None)
        assert y.shape == (2, L, 3) and h.shape == (2, 3, 16), "state shape depends on L"


# --------------------------------------------------------------------------------------
# P12: scaled-identity A (A[d, n] = a[d], the Mamba-2 form of the lesson page's "Mamba-3"
# section).  Every state of a channel then shares the decay, and the product of decays from
# token s+1 to t is exp(a_d (S_t - S_s)) with S_t the running sum of Delta.  Summing the
# unrolled state over n gives y as a masked matrix product over token pairs, with no state
# at all:
#   y_t[d] = sum_{s<=t} exp(a_d (S_t - S_s)) Delta_s x_s <C_t, B_s>  +  exp(a_d S_t) <C_t, h0[d]>
#   h_T[d, n] = sum_s exp(a_d (S_T - S_s)) Delta_s x_s B_s[n]  +  exp(a_d S_T) h0[d, n]
# This is a different algorithm from the recurrence (pairs of tokens, not a walk in time).
# --------------------------------------------------------------------------------------
def scalar_a_dual_form(x, delta, a, B, C, h0):
    batch, L, D = x.shape
    S = np.cumsum(delta, axis=1)                       # inclusive running sums [b, L, D]
    G = np.einsum("btn,bsn->bts", C, B)                # <C_t, B_s>             [b, L, L]
    u = delta * x
    lower = np.tril(np.ones((L, L), dtype=bool))
    y = np.empty((batch, L, D))
    hT = np.empty((batch, D, B.shape[2]))
    for b in range(batch):
        for d in range(D):
            gap = S[b, :, d][:, None] - S[b, :, d][None, :]                # S_t - S_s
            M = np.exp(np.where(lower, a[d] * gap, -np.inf))              # 0 above the diagonal
            y[b, :, d] = (M * G[b]) @ u[b, :, d] + np.exp(a[d] * S[b, :, d]) * (C[b] @ h0[b, d])
            carry = np.exp(a[d] * (S[b, -1, d] - S[b, :, d]))            # [L]
            hT[b, d] = (carry * u[b, :, d]) @ B[b] + np.exp(a[d] * S[b, -1, d]) * h0[b, d]
    return y, hT


def pin_scalar_a_dual_form(impl, seed=13):
    if not hasattr(impl, "prefill_scalar_a"):
        return
    r = _rng(seed)
    batch, L, D, N = 2, 48, 16, 16            # D == N, so a transposed expansion still runs
    x = r.standard_normal((batch, L, D))
    delta = np.logaddexp(0.0, r.standard_normal((batch, L, D)) - 2.0)
    a = -r.integers(1, N + 1, size=D) * r.uniform(0.5, 1.5, size=D)
    B = r.standard_normal((batch, L, N))
    C = r.standard_normal((batch, L, N))
    h0 = r.normal(0.0, 0.5, size=(batch, D, N))
    y, h = impl.prefill_scalar_a(x, delta, a, B, C, h0)
    y_ref, h_ref = scalar_a_dual_form(x, delta, a, B, C, h0)
    assert _rel(y, y_ref) < 1e-12, f"scaled-identity y differs from the dual form {_rel(y, y_ref)}"
    assert _rel(h, h_ref) < 1e-12, f"scaled-identity h differs from the dual form {_rel(h, h_ref)}"
    if hasattr(impl, "step_scalar_a"):
        hs = h0.copy()
        for t in range(L):
            yt, hs = impl.step_scalar_a(hs, x[:, t], delta[:, t], a, B[:, t], C[:, t])
            assert np.array_equal(yt, y[:, t]), f"scaled-identity step y differs at token {t}"
        assert np.array_equal(hs, h), "scaled-identity step chain differs from prefill"


ALL_PINS = [
    pin_brute_force,
    pin_mpmath,
    pin_geometric,
    pin_chunked,
    pin_prefill_equals_steps,
    pin_prefix_sum,
    pin_decay_only,
    pin_scaling,
    pin_causality,
    pin_channel_permutation,
    pin_zero_delta,
    pin_state_shape,
    pin_scalar_a_dual_form,
]


def failing_pins(impl):
    """Names of the pins ``impl`` fails."""
    bad = []
    for p in ALL_PINS:
        try:
            p(impl)
        except (AssertionError, ValueError, IndexError, FloatingPointError) as e:  # noqa: PERF203
            bad.append((p.__name__, str(e)[:80]))
    return bad


# exported for tests that need an exact value of the decay
LOG2E = 1.0 / math.log(2.0)

"""The pins are sharp enough: each plausible mistake planted into a copy of the oracle's
recurrence (written here in numpy, CPU only) fails at least one pin, while the faithful
copy passes all of them."""
import numpy as np
import pytest

import pins


def _make(mistake=None):
    """A numpy copy of the recurrence, optionally carrying one planted mistake."""

    def prefill(x, delta, A, B, C, h0=None):
        x, delta, A, B, C = (np.asarray(v, np.float64) for v in (x, delta, A, B, C))
        batch, L, D = x.shape
        N = A.shape[1]
        h = np.zeros((batch, D, N)) if h0 is None or mistake == "ignore_h0" else np.array(h0, np.float64)
        y = np.zeros((batch, L, D))
        for t in range(L):
            dl = delta[:, t, :, None]                          # [b, D, 1]
            xt = x[:, max(t - 1, 0) if mistake == "stale_x" else t, :, None]
            Bt = B[:, t, None, :]                              # [b, 1, N]
            Ct = C[:, max(t - 1, 0) if mistake == "stale_C" else t, None, :]
            Ad = A[::-1] if mistake == "reversed_A_rows" else A
            if mistake == "shifted_B_index":
                Bt = np.roll(Bt, 1, axis=2)
            if mistake == "wrong_sign":
                abar = np.exp(-dl * Ad[None])
            elif mistake == "exp_of_delta_times_A":
                abar = np.exp(dl) * Ad[None]
            elif mistake == "base_two":
                abar = np.exp2(dl * Ad[None])
            elif mistake == "swapped_x_delta":
                abar = np.exp(xt * Ad[None])
            else:
                abar = np.exp(dl * Ad[None])
            if mistake == "dropped_delta":
                inp = Bt * xt
            else:
                inp = dl * Bt * xt
            h_prev = h
            h = abar * h + inp
            hy = h_prev if mistake == "output_before_update" else h
            terms = Ct * hy
            if mistake == "dropped_state":
                terms = terms[:, :, :-1]
            y[:, t] = terms.sum(axis=2)
        return y, h

    def step(h, x_t, delta_t, A, B_t, C_t):
        y, hn = prefill(np.asarray(x_t)[:, None], np.asarray(delta_t)[:, None], A,
                        np.asarray(B_t)[:, None], np.asarray(C_t)[:, None], h)
        return y[:, 0], hn

    def prefill_chunked(x, delta, A, B, C, chunk, h0=None):
        return prefill(x, delta, A, B, C, h0)

    return type("Impl", (), {"prefill": staticmethod(prefill), "step": staticmethod(step),
                             "prefill_chunked": staticmethod(prefill_chunked)})


MISTAKES = ["ignore_h0", "stale_x", "stale_C", "reversed_A_rows", "shifted_B_index", "wrong_sign",
            "exp_of_delta_times_A", "base_two", "dropped_delta", "swapped_x_delta",
            "output_before_update", "dropped_state"]


def test_faithful_copy_passes_every_pin():
    impl = _make(None)
    bad = [name for name, _ in pins.failing_pins(impl)
           if name not in ("pin_prefill_equals_steps",)]  # numpy sums in another order than step
    assert bad == []


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_mistake_is_caught(mistake):
    with np.errstate(all="ignore"):
        failed = pins.failing_pins(_make(mistake))
    assert failed, f"no pin catches the planted mistake '{mistake}'"

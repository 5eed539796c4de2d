"""The scaled-identity oracle (A[d, n] = a[d]) against pin P12, and the pin's sharpness: a
plausible mistake in turning a into the diagonal A fails it (CPU only)."""
import numpy as np
import pytest

import oracle
import pins


class _Faithful:
    prefill_scalar_a = staticmethod(oracle.prefill_scalar_a)
    step_scalar_a = staticmethod(oracle.step_scalar_a)


def _with_expansion(expand):
    class Impl:
        @staticmethod
        def prefill_scalar_a(x, delta, a, B, C, h0=None):
            return oracle.prefill(x, delta, expand(np.asarray(a, np.float64)), B, C, h0)
    return Impl


MISTAKES = {
    # a[n] down every column instead of a[d] along every row (runs when D == N)
    "transposed": lambda a: np.repeat(a[None, :], 16, axis=0),
    # the diagonal form's per-state factor (n + 1) carried over
    "state_scaled": lambda a: a[:, None] * np.arange(1, 17)[None, :],
    # log2(e) folded in twice, as if A were already the base-2 exponent
    "base_two": lambda a: np.repeat(a[:, None] / np.log(2.0), 16, axis=1),
}


def test_oracle_passes_dual_form():
    pins.pin_scalar_a_dual_form(_Faithful)


def test_faithful_expansion_passes():
    pins.pin_scalar_a_dual_form(_with_expansion(lambda a: np.repeat(a[:, None], 16, axis=1)))


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_pin_catches_mistake(name):
    with pytest.raises(AssertionError):
        pins.pin_scalar_a_dual_form(_with_expansion(MISTAKES[name]))


def test_expand_scalar_a():
    a = np.array([-1.0, -2.5, -0.75])
    A = oracle.expand_scalar_a(a, 16)
    assert A.shape == (3, 16) and np.all(A == a[:, None])
    with pytest.raises(ValueError):
        oracle.expand_scalar_a(np.zeros((2, 2)))

"""The oracle against every pin (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import pins


class _Oracle:
    prefill = staticmethod(oracle.prefill)
    step = staticmethod(oracle.step)
    prefill_scalar_a = staticmethod(oracle.prefill_scalar_a)
    step_scalar_a = staticmethod(oracle.step_scalar_a)

    @staticmethod
    def prefill_chunked(x, delta, A, B, C, chunk, h0=None):
        return oracle.prefill_chunked(x, delta, A, B, C, chunk, h0)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_Oracle)


def test_oracle_threads_do_not_change_bits():
    x, delta, A, B, C, h0 = pins.random_case(21, 3, 50, 11, 16, True)
    y1, h1 = oracle.prefill(x, delta, A, B, C, h0, nthreads=1)
    y7, h7 = oracle.prefill(x, delta, A, B, C, h0, nthreads=7)
    assert np.array_equal(y1, y7) and np.array_equal(h1, h7)


def test_oracle_rejects_bad_shapes():
    x, delta, A, B, C, _ = pins.random_case(22, 1, 5, 3, 16, False)
    with pytest.raises(ValueError):
        oracle.prefill(x, delta[:, :4], A, B, C)
    with pytest.raises(ValueError):
        oracle.prefill(x, delta, A[:2], B, C)
    with pytest.raises(ValueError):
        oracle.prefill(x, delta, A, B[:, :, :3], C)


def _golden(name):
    vals = {}
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = float(v)
    return vals


def test_state_memory_matches_page():
    """The lesson page's memory budget: 28 Mamba layers x hidden 4096 x state 16 x 2 bytes
    is about 3.7 MB, and does not grow with the sequence.  The oracle's state for one layer
    at D = hidden has exactly D * N entries whatever L is."""
    g = _golden("state_memory_lesson_page.txt")
    D, N = int(g["hidden"]), int(g["state_size"])
    for L in (1, 3):
        x = np.zeros((1, L, D))
        _, h = oracle.prefill(x, x, np.zeros((D, N)), np.zeros((1, L, N)), np.zeros((1, L, N)))
        assert h.size == D * N
    total = g["layers"] * h.size * g["bytes_per_value"]
    assert abs(total / 1e6 - g["printed_MB"]) < 0.05

"""Calls on different streams (and from different host threads) run independently: each
result equals the same call made alone.  The library keeps no state between calls, so
nothing here may differ by even one bit."""
import threading

import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import workloads
from gpu_util import bits, say, to_dev

pytestmark = pytest.mark.gpu


def _cases():
    return [to_dev(workloads.small_prefill(1, 1500, 2048, "bf16", seed=s)) for s in (31, 32, 33, 34)]


def test_prefills_on_concurrent_streams_match_serial_calls():
    cases = _cases()
    ref = []
    for c in cases:
        ref.append(jscan.prefill(c["x"], c["delta"], c["A"], c["B"], c["C"]))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    out = []
    for c, s in zip(cases, streams):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            out.append(jscan.prefill(c["x"], c["delta"], c["A"], c["B"], c["C"]))
    torch.cuda.synchronize()
    for (y0, h0), (y1, h1) in zip(ref, out):
        assert torch.equal(bits(y0), bits(y1)) and torch.equal(bits(h0), bits(h1))
    say(f"{len(cases)} prefills on separate streams match")


def test_calls_from_host_threads_match_serial_calls():
    cases = _cases()
    ref = [jscan.prefill(c["x"], c["delta"], c["A"], c["B"], c["C"]) for c in cases]
    torch.cuda.synchronize()
    out = [None] * len(cases)
    errors = []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                c = cases[i]
                out[i] = jscan.prefill(c["x"], c["delta"], c["A"], c["B"], c["C"])
            s.synchronize()
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)

    threads = [threading.Thread(target=work, args=(i,)) for i in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for (y0, h0), (y1, h1) in zip(ref, out):
        assert torch.equal(bits(y0), bits(y1)) and torch.equal(bits(h0), bits(h1))

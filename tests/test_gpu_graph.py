"""jscan_step and jscan_prefill launched inside a captured HIP graph give the same bits as
eager launches, replay after replay (with eager work and synchronisation in between)."""
import pytest
import torch

import mamba_selective_scan_03_amd as jscan
import workloads
from gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


def test_decode_token_step_in_a_graph_matches_eager():
    wl = workloads.Workload("graph_decode", 80, 8, 1, 256, 16, "bf16", True, layers=3)
    layers = [to_dev(workloads.decode_layer_inputs(wl, i)) for i in range(3)]
    h_graph = [L["h0"].clone() for L in layers]
    h_eager = [L["h0"].clone() for L in layers]
    y_graph = [torch.empty_like(L["x"]) for L in layers]
    y_eager = [torch.empty_like(L["x"]) for L in layers]

    def token_step(hs, ys):
        for L, h, y in zip(layers, hs, ys):
            jscan.step(h, L["x"], L["delta"], L["A"], L["B"], L["C"], y_t=y)

    # warm up on a side stream (the binding launches on the current stream), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = [h.clone() for h in h_graph]
        token_step(warm, [torch.empty_like(y) for y in y_graph])
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    snapshot = [h.clone() for h in h_graph]
    with torch.cuda.graph(g):
        token_step(h_graph, y_graph)
    for h, s in zip(h_graph, snapshot):   # capture does not run the kernels; keep the start state
        h.copy_(s)
    for replay in range(4):
        g.replay()
        token_step(h_eager, y_eager)      # eager launches between replays
        torch.cuda.synchronize()
        for i in range(3):
            assert torch.equal(bits(h_graph[i]), bits(h_eager[i])), f"replay {replay} layer {i}: state"
            assert torch.equal(bits(y_graph[i]), bits(y_eager[i])), f"replay {replay} layer {i}: y"


def test_prefill_in_a_graph_matches_eager():
    d = to_dev(workloads.small_prefill(1, 300, 256, "bf16"))
    y_e, h_e = jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"])
    y_g = torch.empty_like(y_e)
    h_g = torch.empty_like(h_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y_g, h_final=h_g)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        jscan.prefill(d["x"], d["delta"], d["A"], d["B"], d["C"], y=y_g, h_final=h_g)
    for replay in range(3):
        y_g.fill_(float("nan"))
        h_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y_g), bits(y_e)) and torch.equal(bits(h_g), bits(h_e)), f"replay {replay}"

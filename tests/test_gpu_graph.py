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


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_time_parallel_prefill_in_a_graph_matches_eager():
    """Three launches (segment summaries, carry, rescan) sharing a workspace, replayed."""
    d = to_dev(workloads.small_prefill(1, 2000, 256, "bf16", seed=4))
    h0 = torch.randn(1, 256, 16, generator=torch.Generator().manual_seed(2)).cuda() * 0.1
    ws = torch.empty(jscan.chunked_workspace_bytes(1, 2000, 256, 256), dtype=torch.uint8, device="cuda")
    y_e, h_e = jscan.prefill_chunked(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, chunk=256, workspace=ws)
    y_g, h_g = torch.empty_like(y_e), torch.empty_like(h_e)
    g = _capture(lambda: jscan.prefill_chunked(d["x"], d["delta"], d["A"], d["B"], d["C"], h0=h0, y=y_g,
                                               h_final=h_g, chunk=256, workspace=ws))
    for replay in range(3):
        y_g.fill_(float("nan"))
        h_g.fill_(float("nan"))
        ws.fill_(0xAB)                    # the workspace's contents on entry do not matter
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(y_g), bits(y_e)) and torch.equal(bits(h_g), bits(h_e)), f"replay {replay}"


def test_producer_and_fused_prefill_in_a_graph_match_eager():
    x = workloads.small_prefill(1, 512, 256, "bf16", seed=6)
    d = to_dev(x)
    w = {k: v.cuda() for k, v in workloads.producer_weights(256, 256, seed=6).items()}
    _, B_e, C_e, dl_e = jscan.ssm_inputs(d["x"], w["w_x"], w["g_d"], w["g_b"], w["g_c"], w["w_dt"], w["b_dt"],
                                         skip_delta=True)
    y_e, h_e = jscan.prefill_fused(d["x"], dl_e, w["w_dt"], w["b_dt"], d["A"], B_e, C_e)
    B_g, C_g, dl_g = torch.empty_like(B_e), torch.empty_like(C_e), torch.empty_like(dl_e)
    y_g, h_g = torch.empty_like(y_e), torch.empty_like(h_e)

    def layer():
        jscan.ssm_inputs(d["x"], w["w_x"], w["g_d"], w["g_b"], w["g_c"], w["w_dt"], w["b_dt"], B=B_g, C=C_g,
                         delta_low=dl_g, skip_delta=True)
        jscan.prefill_fused(d["x"], dl_g, w["w_dt"], w["b_dt"], d["A"], B_g, C_g, y=y_g, h_final=h_g)
    g = _capture(layer)
    for replay in range(3):
        for t in (B_g, C_g, dl_g, y_g):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in ((B_g, B_e), (dl_g, dl_e), (y_g, y_e), (h_g, h_e)):
            assert torch.equal(bits(got), bits(want)), f"replay {replay}"

"""HIP graph capture of the layer's entry points.

moe_forward and moe_backward enqueue kernels only (no allocation, no
memset, no synchronisation, no host read-back), so a caller can capture
them once in a HIP graph and replay it.  Each replay, with the program's own
eager work and synchronisations between replays, must reproduce the eager
call's bits: y and the routing/dispatch outputs of the forward, every
gradient of the backward.
"""
import pytest
import torch

from top_routing_expert_route_amd import api
from top_routing_expert_route_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = {
    "drop-small": wl.scaled(wl.get(2), name="drop-small", T=1000, d=192, ffn=256),
    "dsv3-small": wl.scaled(wl.get(4), name="dsv3-small", T=500, d=192, ffn=256, expert_begin=32,
                            expert_bias="gauss"),
    "tiny-fp32": wl.get(0),
}


def _bits(a):
    if a.dtype == torch.bfloat16:
        return a.view(torch.int16)
    return a.view(torch.int32) if a.dtype == torch.float32 else a


@pytest.mark.parametrize("name", list(CASES))
def test_forward_and_backward_graph_replays(name):
    w = CASES[name]
    print("graph case", name, flush=True)
    inp = wl.make_layer(w, seed=5)
    t = wl.device_layer(inp, DEV)
    dy = wl.to_torch(wl.make_grad_output(w, seed=5), DEV)
    dt = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32
    layer = api.Layer(w.T, w.d, w.E, w.k, w.ffn, dt, w.capacity_factor, w.expert_begin, w.num_local_experts,
                      w.alpha, t["w_router"], t["b_router"], t["w1"], t["b1"], t["w2"], t["b2"], t["ws1"],
                      t["bs1"], t["ws2"], t["bs2"], device=DEV, sel_bias=t["sel_bias"])
    outs = layer.alloc_outputs()
    x = t["x"]
    y_ref = layer.forward(x).clone()
    o_ref = {k: v.clone() for k, v in outs.items()}
    grads = layer.backward(x, dy, 0.7)
    torch.cuda.synchronize()
    g_ref = {k: v.clone() for k, v in grads.items()}
    y = torch.empty_like(y_ref)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, y)
        layer.backward(x, dy, 0.7, grads=grads)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer.forward(x, y)
        layer.backward(x, dy, 0.7, grads=grads)

    for _ in range(3):
        y.fill_(3.0)
        outs["topk_idx"].fill_(-1)
        outs["slot_row"].fill_(-7)
        for v in grads.values():
            v.fill_(5.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref))
        for k in ("topk_idx", "topk_w", "seg_offsets", "slot_row", "f", "P", "l_aux"):
            assert torch.equal(_bits(outs[k]), _bits(o_ref[k])), k
        for k in g_ref:
            assert torch.equal(_bits(grads[k]), _bits(g_ref[k])), k


def test_overlap_forward_graph_replays():
    """moe_forward_overlap captured with its side stream and fork/join events:
    every replay reproduces the eager moe_forward bits."""
    w = CASES["dsv3-small"]
    inp = wl.make_layer(w, seed=6)
    t = wl.device_layer(inp, DEV)
    layer = api.Layer(w.T, w.d, w.E, w.k, w.ffn, torch.bfloat16, w.capacity_factor, w.expert_begin,
                      w.num_local_experts, w.alpha, t["w_router"], t["b_router"], t["w1"], t["b1"], t["w2"],
                      t["b2"], t["ws1"], t["bs1"], t["ws2"], t["bs2"], device=DEV, sel_bias=t["sel_bias"])
    outs = layer.alloc_outputs()
    x = t["x"]
    y_ref = layer.forward(x).clone()
    o_ref = {k: v.clone() for k, v in outs.items()}
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    cap = torch.cuda.Stream()
    side = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        layer.forward(x, y, side_stream=side)  # warm-up on the capture stream (events created here)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y_ref))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        layer.forward(x, y, side_stream=side)
    for _ in range(3):
        y.fill_(3.0)
        outs["topk_idx"].fill_(-1)
        outs["slot_row"].fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(y_ref))
        for k in ("topk_idx", "topk_w", "seg_offsets", "slot_row", "f", "P", "l_aux"):
            assert torch.equal(_bits(outs[k]), _bits(o_ref[k])), k

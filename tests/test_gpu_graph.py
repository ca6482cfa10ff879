"""The layer captured in a HIP graph (torch.cuda.CUDAGraph over the library's launches):
replays with new inputs copied into the captured buffers give, bit for bit, what eager
calls give on the same inputs -- several replays in a row, with eager work and
synchronisation between them. (The library's per-call state lives in the kernels: the plan
clears the tile flags, dispatch raises them with the captured epoch.)"""
import pytest
import torch

import combine_moe_dispatch_02_amd as moe
from synth import config_by_name, MoEConfig, make_inputs

from _gpu import dev_inputs, make_layer, say

pytestmark = pytest.mark.gpu

GRAPH_CASES = [
    config_by_name("tiny"),
    MoEConfig("graph_big", 600, 1024, 512, 8, 0, 8, 4, 128),           # big-tile kernels, ring
    MoEConfig("graph_fp8", 300, 512, 256, 6, 0, 6, 2, 64, "fp8"),
]


@pytest.mark.parametrize("cfg", GRAPH_CASES, ids=[c.name for c in GRAPH_CASES])
def test_layer_graph_replays_match_eager(cfg):
    base = dev_inputs(make_inputs(cfg))
    layer = make_layer(cfg)
    w = layer.prepare_weights(base["w1"], base["w2"], base["w1s"], base["w2s"])
    x, idx, tw = base["x"].clone(), base["idx"].clone(), base["w"].clone()
    say("graph capture", cfg.name)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.forward(x, idx, tw, *w)                   # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer.forward(x, idx, tw, *w)
    eager = make_layer(cfg)
    for i in range(4):
        inp = dev_inputs(make_inputs(cfg, seed=1000 + i))
        x.copy_(inp["x"])
        idx.copy_(inp["idx"])
        tw.copy_(inp["w"])
        g.replay()
        torch.cuda.synchronize()
        ref = eager.forward(inp["x"], inp["idx"], inp["w"], *w).clone()
        torch.cuda.synchronize()
        assert moe.moe_get_error(layer.ws) == 0 and moe.moe_get_error(eager.ws) == 0
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i}"

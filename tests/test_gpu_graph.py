"""The layer inside a HIP graph: moe_exl3_layer only launches kernels on the
caller's stream (no allocation, copy, memset or synchronisation), so a
captured call replays.  Each replay is checked bit for bit against an eager
call on the same inputs, with eager work and device synchronisations between
the replays, and the input's contents are changed in place before the last
replay (the graph reads the buffers, not the values seen at capture)."""
import numpy as np
import pytest
import torch

import trellis_quantized_moe_exl3_amd as M
import workloads as W
from gpu_util import DevLayer

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,T", [("decode", 8), ("decode", 300)])
def test_layer_graph_replays_match_eager(name, T):
    # 8 tokens: single-block routing tail, GEMV with the shared expert's
    # blocks; 300 tokens: multi-launch routing, MFMA tiles with the shared
    # expert's dense tiles
    cfg = W.BY_NAME[name].replace(tokens=T, router_bias=True)
    inp = W.gen_layer(cfg)
    dl = DevLayer(inp)
    x = dl.x.clone()
    ws = dl.workspace(T)
    out_g = torch.empty_like(x)

    def eager(xin):
        o = torch.empty_like(xin)
        M.layer(dl.desc, dl.weights, xin, o, dl.workspace(T))
        torch.cuda.synchronize()
        return o.clone()

    ref = eager(x)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up call on the capture stream
        M.layer(dl.desc, dl.weights, x, out_g, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.layer(dl.desc, dl.weights, x, out_g, ws)
    torch.cuda.synchronize()

    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # eager work between replays, on other buffers
        other = eager(x.flip(0).contiguous())
        assert other.shape == x.shape

    # new activations in place: the replay follows them
    x.copy_(x.flip(0))
    torch.cuda.synchronize()
    ref2 = eager(x)
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(out_g.view(torch.int16), ref2.view(torch.int16))
    assert not torch.equal(ref2.view(torch.int16), ref.view(torch.int16))
    del g

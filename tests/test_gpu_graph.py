"""GPU: the layer captured into a HIP graph and replayed. Every replay, with eager layer
calls and a change of the input in between, must give exactly the eager result for the
input the graph's buffers hold at that moment."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
from parity import bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host, make_shared_host

pytestmark = pytest.mark.gpu

# 300 tokens over 4 experts: 150 rows per expert, several tiles at every height
CFG = Config("graph", 300, 256, 256, 4, 2, "normal", "uniform", "softmax", True, seed=21)


@pytest.mark.parametrize("flags", [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224],
                         ids=["auto", "16", "128", "192", "224"])
def test_layer_replays_in_a_hip_graph(flags):
    x_bits = make_x_bits(CFG)
    x2_bits = make_x_bits(CFG, seed=22)
    ids, w = make_routing(CFG)
    exd = experts_dev(make_experts_host(CFG))
    shd = experts_dev(make_shared_host(CFG))
    x = bf16_dev(x_bits)
    x2 = bf16_dev(x2_bits)
    t_ids = torch.from_numpy(ids).cuda()
    t_w = torch.from_numpy(w).cuda()

    say(f"graph eager flags={flags}")
    eager = bits_host(moe.moe_layer(x, t_ids, t_w, exd, shd, flags=flags))
    eager2 = bits_host(moe.moe_layer(x2, t_ids, t_w, exd, shd, flags=flags))
    torch.cuda.synchronize()

    say(f"graph capture flags={flags}")
    x_in = x.clone()                      # the buffer the graph reads
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):         # warm-up on the capture stream
        moe.moe_layer(x_in, t_ids, t_w, exd, shd, flags=flags)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = moe.moe_layer(x_in, t_ids, t_w, exd, shd, flags=flags)
    torch.cuda.synchronize()

    for rep in range(4):
        say(f"graph replay {rep} flags={flags}")
        src, want = (x, eager) if rep % 2 == 0 else (x2, eager2)
        x_in.copy_(src)
        # eager work of the same shapes between replays, sharing the cached workspaces
        other = moe.moe_layer(x2 if rep % 2 == 0 else x, t_ids, t_w, exd, shd, flags=flags)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(out), want), f"replay {rep} differs from the eager result"
        assert np.array_equal(bits_host(other), eager2 if rep % 2 == 0 else eager)

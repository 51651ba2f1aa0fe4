"""GPU: layers on two streams at once. Each stream gets workspaces of its own from the binding,
so two batches run concurrently must give exactly what each gives alone (the layer is
deterministic: the same bits every time)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
from parity import bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host, make_shared_host

pytestmark = pytest.mark.gpu

# two batches of different sizes through the same experts (so both use many-row tiles), with
# a shared expert (which runs on the binding's own side stream)
CFG_A = Config("streams_a", 600, 512, 512, 8, 2, "normal", "uniform", "softmax", True, seed=101)
CFG_B = Config("streams_b", 350, 512, 512, 8, 2, "normal", "uniform", "softmax", True, seed=102)


def test_two_streams_give_the_results_of_one():
    exd = experts_dev(make_experts_host(CFG_A))
    shd = experts_dev(make_shared_host(CFG_A))
    inputs = []
    for cfg in (CFG_A, CFG_B):
        ids, w = make_routing(cfg)
        inputs.append((bf16_dev(make_x_bits(cfg)), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()))
    say("streams: each batch alone")
    alone = [bits_host(moe.moe_layer(x, i, w, exd, shd)) for x, i, w in inputs]
    torch.cuda.synchronize()

    say("streams: both batches at once, 8 rounds")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    main = torch.cuda.current_stream()
    s1.wait_stream(main)
    s2.wait_stream(main)
    outs = ([], [])
    for _ in range(8):
        for k, s in enumerate((s1, s2)):
            with torch.cuda.stream(s):
                x, i, w = inputs[k]
                outs[k].append(moe.moe_layer(x, i, w, exd, shd))
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    for k in range(2):
        for r, o in enumerate(outs[k]):
            assert np.array_equal(bits_host(o), alone[k]), f"batch {k}, round {r}: differs from the batch alone"

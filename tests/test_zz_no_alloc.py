"""GPU: moe_grouped_swiglu_noalloc (no workspace argument: the library's fixed per-GPU scratch
array holds the intermediates) against moe_grouped_swiglu with a caller workspace, bit for bit,
on two calls in a row, the second with a smaller input (so stale contents of the array from the
first call must not matter), at every tile height; and the host-side rejection of a problem
whose workspace would exceed MOE_NOALLOC_SCRATCH_BYTES."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
from mixture_experts_ffn_ids_amd import _lib as moe_lib
from mixture_experts_ffn_ids_amd._lib import MoeError
from parity import bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host

pytestmark = pytest.mark.gpu

NOALLOC_BYTES = 64 << 20
BIG = Config("noalloc_big", 600, 1024, 512, 12, 4, "rmsnorm", "uniform", "uniform", False, seed=91)
SMALL = Config("noalloc_small", 37, 1024, 512, 12, 2, "normal", "uniform", "uniform", False, seed=92)
TILES = [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224, moe.FLAG_TILE_256]


def _case(cfg):
    x = bf16_dev(make_x_bits(cfg))
    ids, _ = make_routing(cfg)
    return x, moe.dispatch(torch.from_numpy(ids).cuda(), cfg.E)


def test_noalloc_matches_the_workspace_call_on_two_calls_in_a_row():
    exd = experts_dev(make_experts_host(BIG))          # both configs use the same 12 experts
    cases = [_case(BIG), _case(SMALL)]
    for flags in TILES:
        for cfg, (x, disp) in zip((BIG, SMALL), cases):
            say(f"noalloc {cfg.name} N={cfg.N} K={cfg.K} flags={flags}")
            got = bits_host(moe.grouped_swiglu_noalloc(x, disp, exd, flags))
            ref = bits_host(moe.grouped_swiglu(x, disp, exd, flags))
            torch.cuda.synchronize()
            assert np.array_equal(got, ref), f"{cfg.name} flags={flags}"


def test_noalloc_rejects_problems_beyond_its_scratch():
    lib = moe_lib.lib()
    # at K2 shapes a 4096-token batch needs more than the fixed scratch, 256 tokens fit
    assert lib.moe_swiglu_workspace_size(4096, 8, 384, 7168, 2048) > NOALLOC_BYTES
    assert lib.moe_swiglu_workspace_size(256, 8, 384, 7168, 2048) <= NOALLOC_BYTES
    # one expert of intermediate size 65536 over 4096 tokens: h alone is 256 MiB. The call is
    # rejected on the host before anything is enqueued, so the weights need no values.
    N, d, d_ff = 4096, 256, 65536
    assert lib.moe_swiglu_workspace_size(N, 1, 1, d, d_ff) > NOALLOC_BYTES

    class Ex:
        pass

    ex = Ex()
    ex.w_gate = torch.empty((1, d_ff, d), dtype=torch.uint8, device="cuda")
    ex.w_up = torch.empty((1, d_ff, d), dtype=torch.uint8, device="cuda")
    ex.w_down = torch.empty((1, d, d_ff), dtype=torch.uint8, device="cuda")
    ex.s_gate = torch.empty((1, d_ff // 128, d // 128), dtype=torch.float32, device="cuda")
    ex.s_up = torch.empty((1, d_ff // 128, d // 128), dtype=torch.float32, device="cuda")
    ex.s_down = torch.empty((1, d // 128, d_ff // 128), dtype=torch.float32, device="cuda")
    x = torch.zeros((N, d), dtype=torch.bfloat16, device="cuda")
    disp = moe.identity_dispatch(N, x.device)
    say("noalloc beyond its scratch (host-side rejection)")
    with pytest.raises(MoeError) as err:
        moe.grouped_swiglu_noalloc(x, disp, ex)
    assert err.value.status == 4    # MOE_ERR_WORKSPACE

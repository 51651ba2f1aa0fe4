"""GPU: the top-1 experts with the combine done by the down projection's epilogue
(moe_grouped_swiglu_top1) against the unfused calls (moe_grouped_swiglu, then moe_combine with
K = 1), bit for bit, and against the oracle within the layer tolerance."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import assert_layer_close, bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host

pytestmark = pytest.mark.gpu

TILES = [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224, moe.FLAG_TILE_256]
TILE_IDS = ["auto", "16", "128", "192", "224", "256"]
# 700 rows over 5 experts: several row tiles per expert at every tile height, ragged last tiles;
# d = 640 is two and a half 256-column output blocks (a ragged last block). d_ff = 2048, the
# experts' size: with one choice per token nothing averages the matrix cores' accumulation
# error over experts, and at d_ff = 1024 one token's relative L2 reached 1.15e-2
CFG = Config("top1", 700, 640, 2048, 5, 1, "normal", "uniform", "ones", False, seed=71)


# d_ff = 1024 with one choice per token: with gate|up's block sums on the FP8 matrix ops (which
# round their internal sums) one token's relative L2 reached 1.15e-2 here, over the bar; with the
# exact block sums every tile height must hold it
CFG_1024 = Config("top1_dff1024", 700, 640, 1024, 5, 1, "normal", "uniform", "ones", False, seed=71)


def _case(cfg=CFG):
    x = make_x_bits(cfg)
    ids, _ = make_routing(cfg)
    # weights of both signs, some zero, not normalised: the epilogue applies them as the combine does
    w = np.random.default_rng(72).uniform(-2.0, 2.0, (cfg.N, 1)).astype(np.float32)
    w[::97] = 0.0
    return x, ids, w, make_experts_host(cfg)


def _unfused(x_d, disp, w_d, exd, flags):
    y = moe.grouped_swiglu(x_d, disp, exd, flags)
    return moe.combine(y, disp, w_d)


@pytest.mark.parametrize("flags", TILES, ids=TILE_IDS)
def test_top1_matches_unfused_and_oracle(flags):
    x, ids, w, exh = _case()
    exd = experts_dev(exh)
    x_d, w_d = bf16_dev(x), torch.from_numpy(w).cuda()
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), CFG.E)
    say(f"top1 N={CFG.N} d={CFG.d} E={CFG.E} flags={flags}")
    fused = bits_host(moe.grouped_swiglu_top1(x_d, disp, w_d, exd, flags))
    ref = bits_host(_unfused(x_d, disp, w_d, exd, flags))
    torch.cuda.synchronize()
    assert np.array_equal(fused, ref)
    _, ref64 = oracle.moe_forward(x, ids, w, exh)
    assert_layer_close(fused, ref64, f"top1 flags={flags}")


@pytest.mark.parametrize("flags", TILES, ids=TILE_IDS)
def test_top1_small_dff_within_tolerance(flags):
    x, ids, w, exh = _case(CFG_1024)
    exd = experts_dev(exh)
    x_d, w_d = bf16_dev(x), torch.from_numpy(w).cuda()
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), CFG_1024.E)
    say(f"top1 d_ff=1024 N={CFG_1024.N} flags={flags}")
    out = bits_host(moe.grouped_swiglu_top1(x_d, disp, w_d, exd, flags))
    torch.cuda.synchronize()
    _, ref64 = oracle.moe_forward(x, ids, w, exh)
    assert_layer_close(out, ref64, f"top1 d_ff=1024 flags={flags}")


def test_moe_layer_top1_uses_the_fused_path():
    x, ids, w, exh = _case()
    exd = experts_dev(exh)
    x_d, w_d, ids_d = bf16_dev(x), torch.from_numpy(w).cuda(), torch.from_numpy(ids).cuda()
    say("moe_layer K=1")
    moe.profile_reset()
    moe.profile_enable(True)
    out = bits_host(moe.moe_layer(x_d, ids_d, w_d, exd))
    torch.cuda.synchronize()
    moe.profile_enable(False)
    assert moe.profile_read(moe.KERNEL_COMBINE)[1] == 0      # no separate combine launch
    assert np.array_equal(out, bits_host(_unfused(x_d, moe.dispatch(ids_d, CFG.E), w_d, exd, 0)))


def test_top1_empty_and_dropped_tokens():
    x, ids, w, exh = _case()
    exd = experts_dev(exh)
    say("top1 N=0")
    empty = torch.empty((0, CFG.d), dtype=torch.bfloat16, device="cuda")
    d0 = moe.dispatch(torch.empty((0, 1), dtype=torch.int32, device="cuda"), CFG.E)
    assert tuple(moe.grouped_swiglu_top1(empty, d0, torch.empty((0, 1), device="cuda"), exd).shape) == (0, CFG.d)
    # ids out of range (fast-mode dispatch leaves those tokens out): their out rows become +0,
    # as the unfused combine gives a token with no valid choice; every row matches the unfused
    # result bit for bit, whatever out held before
    bad = ids.copy()
    bad[[3, 250, 699]] = CFG.E + 1
    bad[500] = -1
    x_d, w_d = bf16_dev(x), torch.from_numpy(w).cuda()
    disp = moe.dispatch(torch.from_numpy(bad).cuda(), CFG.E)
    ref = bits_host(_unfused(x_d, disp, w_d, exd, 0))
    for flags in (0, moe.FLAG_TILE_16, moe.FLAG_TILE_192):
        out = torch.full((CFG.N, CFG.d), 7.0, dtype=torch.bfloat16, device="cuda")
        say(f"top1 dropped tokens flags={flags}")
        moe.grouped_swiglu_top1(x_d, disp, w_d, exd, flags, out=out)
        torch.cuda.synchronize()
        got = bits_host(out)
        assert np.array_equal(got, ref)
        assert np.all(got[[3, 250, 500, 699]] == 0)


def test_moe_layer_top1_dropped_token_is_zero():
    """moe_layer with K = 1 and an out-of-range id (fast mode) returns +0 for that token and the
    unfused result everywhere, not whatever the fresh output buffer held."""
    x, ids, w, exh = _case()
    exd = experts_dev(exh)
    bad = ids.copy()
    bad[[0, 17]] = CFG.E + 3
    x_d, w_d, ids_d = bf16_dev(x), torch.from_numpy(w).cuda(), torch.from_numpy(bad).cuda()
    # fill the caching allocator's free blocks with non-zero bytes first, so that a row left
    # unwritten would show
    junk = torch.full((CFG.N * CFG.d * 4,), 0x7F, dtype=torch.uint8, device="cuda")
    del junk
    say("moe_layer K=1 with out-of-range ids")
    out = bits_host(moe.moe_layer(x_d, ids_d, w_d, exd))
    torch.cuda.synchronize()
    ref = bits_host(_unfused(x_d, moe.dispatch(ids_d, CFG.E), w_d, exd, 0))
    assert np.array_equal(out, ref)
    assert np.all(out[[0, 17]] == 0)

"""GPU: the dense block's SwiGLU MLP run through the grouped kernels as one expert that every
token visits (E = 1, K = 1, weight 1), against the oracle. For that routing the oracle's layer
is the MLP forward of the "SwiGLU output" page, down(silu(gate x) * up x), a reduction the
oracle's own pins check. Outputs are held to the layer tolerance."""
import functools

import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import assert_layer_close, bf16_dev, bits_host, experts_dev, say
from workloads import Config, config_by_name, make_routing, make_x_bits
from workloads.gen import experts_to_host, make_block_inputs, make_experts_device, make_experts_host

pytestmark = pytest.mark.gpu

EPS = 1e-6
# 500 rows: several row tiles at every tile height, each with a ragged last tile; d_ff = 1152
# is nine 128-column requantisation groups, d = 1024 eight down column blocks
SMALL = Config("dense_small", 500, 1024, 1152, 1, 1, "normal", "uniform", "ones", False, seed=61, dense=True)
TILES = [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224, moe.FLAG_TILE_256]
TILE_IDS = ["auto", "16", "128", "192", "224", "256"]


@functools.lru_cache(maxsize=None)
def _small_case():
    x = make_x_bits(SMALL)
    ids, w = make_routing(SMALL)
    assert np.all(ids == 0) and np.all(w == 1.0)
    exh = make_experts_host(SMALL)
    _, ref64 = oracle.moe_forward(x, ids, w, exh)
    return x, ids, w, exh, ref64


@pytest.mark.parametrize("flags", TILES, ids=TILE_IDS)
def test_dense_mlp_against_oracle(flags):
    x, ids, w, exh, ref64 = _small_case()
    exd = experts_dev(exh)
    say(f"dense_swiglu N={SMALL.N} d={SMALL.d} d_ff={SMALL.d_ff} flags={flags}")
    out = moe.dense_swiglu(bf16_dev(x), exd, flags)
    torch.cuda.synchronize()
    got = bits_host(out)
    assert_layer_close(got, ref64, f"dense flags={flags}")
    # the routed layer call with the same single expert gives the same bits (its combine of one
    # unit-weight choice adds a bfloat16 value to zero exactly)
    say(f"moe_layer as dense flags={flags}")
    out2 = moe.moe_layer(bf16_dev(x), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), exd, flags=flags)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out2), got)


def test_dense_block_ffn_against_oracle():
    cfg = SMALL
    h_bits, _ = make_block_inputs(cfg)
    g_bits = torch.from_numpy(np.random.default_rng(62).uniform(0.5, 1.5, cfg.d).astype(np.float32)) \
        .to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ids, w = make_routing(cfg)
    exh = make_experts_host(cfg)
    x_norm = oracle.rmsnorm_rows(h_bits, g_bits, EPS)
    _, ref64 = oracle.moe_forward(x_norm, ids, w, exh, residual=h_bits)
    exd = experts_dev(exh)
    outs = []
    for flags in (0, moe.FLAG_TILE_16, moe.FLAG_TILE_256):
        say(f"dense_block_ffn flags={flags}")
        out = moe.dense_block_ffn(bf16_dev(h_bits), bf16_dev(g_bits), EPS, exd, flags)
        torch.cuda.synchronize()
        outs.append(bits_host(out))
        assert_layer_close(outs[-1], ref64, f"dense block flags={flags}")
    # in place on the residual stream: the same bits as the out-of-place call
    h = bf16_dev(h_bits)
    say("dense_block_ffn in place")
    moe.dense_block_ffn(h, bf16_dev(g_bits), EPS, exd, out=h)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(h), outs[0])


def test_dense_empty_and_rejects_routed_sets():
    exd = experts_dev(_small_case()[3])
    say("dense_swiglu N=0")
    out = moe.dense_swiglu(torch.empty((0, SMALL.d), dtype=torch.bfloat16, device="cuda"), exd)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, SMALL.d)
    two = make_experts_host(Config("two", 4, 256, 128, 2, 1, "normal", "uniform", "ones", False, seed=63))
    with pytest.raises(ValueError):
        moe.dense_swiglu(torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda"), experts_dev(two))


def test_dense_block_full_size():
    """The dense block (hidden + MLP(RMSNorm(hidden))) at its benchmark shape (8192 tokens,
    d = 7168, d_ff = 18432) in the launch configuration the benchmark times; outputs on 256
    tokens: both ends, both sides of several 192-row tile edges and random ones. (The MLP alone
    is compared on every token in test_gpu_whole_batch.py.)"""
    cfg = config_by_name("k2_dense_8192")
    ids, w = make_routing(cfg)
    say("dense full-size weights")
    exd = make_experts_device(cfg)
    edges = [t for e in range(192, cfg.N, 192 * 7) for t in (e - 1, e)]
    tok = np.array(sorted({0, 1, 4095, cfg.N - 1, *edges} |
                          set(np.random.default_rng(64).choice(cfg.N, 256 - 4 - len(edges),
                                                               replace=False).tolist())), np.int64)
    exh = experts_to_host(exd)
    h_bits, g_bits = make_block_inputs(cfg)
    say("dense full-size block")
    blk = bits_host(moe.dense_block_ffn(bf16_dev(h_bits), bf16_dev(g_bits), EPS, exd))
    say(f"dense full-size block oracle tokens={len(tok)}")
    x_norm = oracle.rmsnorm_rows(h_bits[tok], g_bits, EPS)
    _, ref_blk = oracle.moe_forward(x_norm, ids[tok], w[tok], exh, residual=h_bits[tok])
    assert_layer_close(blk[tok], ref_blk, f"dense block full size, {len(tok)} tokens")

"""GPU: the layer's neighbours fused in (the block's RMSNorm into the activation quantisation,
its residual addition into the combine) against the oracle.

The fused RMSNorm takes the oracle's steps in the same precisions, so the normalised rows, the
e4m3 codes and the scales are compared bit for bit. (Only the order of the double-precision sum
of squares differs; it changes the float32 mean only if that sum falls within about 2^-53 of a
float32 rounding midpoint.) Layer outputs are held to the layer tolerance."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import assert_layer_close, bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing
from workloads.gen import make_block_inputs, make_experts_host, make_shared_host

pytestmark = pytest.mark.gpu

EPS = 1e-6


def _bf16(v) -> np.ndarray:
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(37, 7168), (5, 128), (3, 65536), (300, 384)])
def test_rmsnorm_quantize_bit_exact(rows, cols):
    rng = np.random.default_rng(rows + cols)
    h = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-8, 8, (rows, 1)))
    h[0] = 0.0                               # a zero row: eps keeps it finite
    if rows > 1:
        h[1] = 2.5                           # a constant row
    h_bits = _bf16(h)
    g_bits = _bf16(rng.uniform(0.25, 2.0, cols))
    say(f"rmsnorm_quantize rows={rows} cols={cols}")
    q, s, y = moe.rmsnorm_quantize(bf16_dev(h_bits), bf16_dev(g_bits), EPS, keep_normed=True)
    torch.cuda.synchronize()
    y_ref = oracle.rmsnorm_rows(h_bits, g_bits, EPS)
    q_ref, s_ref = oracle.quant_rows_bf16(y_ref)
    assert np.array_equal(bits_host(y), y_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    # without the normalised rows the codes and scales are the same
    q2, s2, y2 = moe.rmsnorm_quantize(bf16_dev(h_bits), bf16_dev(g_bits), EPS)
    torch.cuda.synchronize()
    assert y2 is None and torch.equal(q2, q) and torch.equal(s2, s)


@pytest.mark.parametrize("flags", [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224,
                                   moe.FLAG_TILE_256], ids=["auto", "16", "128", "192", "224", "256"])
def test_grouped_swiglu_on_quantised_input_matches(flags):
    cfg = Config("q_in", 200, 384, 256, 5, 2, "normal", "uniform", "softmax", False, seed=51)
    from workloads import make_x_bits
    x = bf16_dev(make_x_bits(cfg))
    ids, _ = make_routing(cfg)
    exd = experts_dev(make_experts_host(cfg))
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), cfg.E)
    say(f"grouped_swiglu_q flags={flags}")
    y_ref = moe.grouped_swiglu(x, disp, exd, flags)
    xq, xs = moe.quantize_rows(x)
    y_q = moe.grouped_swiglu_q(xq, xs, disp, exd, flags)
    torch.cuda.synchronize()
    assert torch.equal(y_q.view(torch.int16), y_ref.view(torch.int16))


def _block_case(cfg, with_shared):
    h_bits, g_bits = make_block_inputs(cfg)
    ids, w = make_routing(cfg)
    exh = make_experts_host(cfg)
    shh = make_shared_host(cfg) if with_shared else None
    return h_bits, g_bits, ids, w, exh, shh


@pytest.mark.parametrize("with_shared", [False, True], ids=["routed", "shared"])
def test_block_ffn_against_oracle(with_shared):
    cfg = Config("block", 77, 384, 1024, 6, 3, "normal", "uniform", "dirichlet", with_shared, seed=52)
    h_bits, g_bits, ids, w, exh, shh = _block_case(cfg, with_shared)
    g_bits = _bf16(np.random.default_rng(53).uniform(0.5, 1.5, cfg.d))
    x_norm = oracle.rmsnorm_rows(h_bits, g_bits, EPS)
    _, ref64 = oracle.moe_forward(x_norm, ids, w, exh, shh, residual=h_bits)
    exd = experts_dev(exh)
    shd = experts_dev(shh) if shh is not None else None
    h = bf16_dev(h_bits)
    t_ids, t_w = torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    outs = []
    for flags in (0, moe.FLAG_TILE_16, moe.FLAG_TILE_128):
        say(f"block_ffn shared={with_shared} flags={flags}")
        out = moe.moe_block_ffn(h, bf16_dev(g_bits), EPS, t_ids, t_w, exd, shd, flags=flags)
        torch.cuda.synchronize()
        outs.append(bits_host(out))
        assert_layer_close(outs[-1], ref64, f"block {'shared' if with_shared else 'routed'} flags={flags}")
        assert np.array_equal(outs[-1], outs[0])
    # the residual stream updated in place gives the same bits
    h2 = bf16_dev(h_bits)
    say("block_ffn in place")
    moe.moe_block_ffn(h2, bf16_dev(g_bits), EPS, t_ids, t_w, exd, shd, out=h2)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(h2), outs[0])


def test_combine_residual_zero_weights_returns_residual():
    cfg = Config("res0", 40, 256, 128, 4, 2, "normal", "uniform", "softmax", False, seed=54)
    h_bits, _ = make_block_inputs(cfg)
    ids, w = make_routing(cfg)
    exd = experts_dev(make_experts_host(cfg))
    h = bf16_dev(h_bits)
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), cfg.E)
    y = moe.grouped_swiglu(h, disp, exd)
    say("combine residual, zero weights")
    out = moe.combine(y, disp, torch.zeros_like(torch.from_numpy(w)).cuda(), residual=h)
    torch.cuda.synchronize()
    assert np.array_equal(bits_host(out), h_bits)

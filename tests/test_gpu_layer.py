"""GPU: the whole layer (moe_dispatch -> moe_grouped_swiglu -> moe_combine) against the
oracle, element by element, within the layer tolerance; plus bit-identity across tile
shapes and across runs (no float atomics anywhere)."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import assert_layer_close, bf16_dev, bits_host, experts_dev, say
from workloads import CONFIGS, Config, make_routing, make_x_bits
from workloads.gen import make_experts_host, make_shared_host

pytestmark = pytest.mark.gpu

SHAPES = {"16": moe.FLAG_TILE_16, "128": moe.FLAG_TILE_128, "192": moe.FLAG_TILE_192, "224": moe.FLAG_TILE_224,
          "256": moe.FLAG_TILE_256}


def _layer(x_bits, ids, w, ex_dev, sh_dev=None, flags=0):
    x = bf16_dev(x_bits)
    t_ids = torch.from_numpy(ids).cuda()
    t_w = torch.from_numpy(w).cuda()
    out = moe.moe_layer(x, t_ids, t_w, ex_dev, sh_dev, flags=flags)
    torch.cuda.synchronize()
    return bits_host(out)


def _check_small(cfg: Config, ids=None, w=None, shapes=("auto", "16", "128", "192", "224", "256")):
    x = make_x_bits(cfg)
    if ids is None:
        ids, w = make_routing(cfg)
    exh = make_experts_host(cfg)
    shh = make_shared_host(cfg) if cfg.shared else None
    ref_bits, ref64 = oracle.moe_forward(x, ids, w, exh, shh)
    exd = experts_dev(exh)
    shd = experts_dev(shh) if shh is not None else None
    outs = {}
    for shape in shapes:
        say(f"layer {cfg.name} N={cfg.N} d={cfg.d} d_ff={cfg.d_ff} E={cfg.E} K={cfg.K} shape={shape}")
        outs[shape] = _layer(x, ids, w, exd, shd, 0 if shape == "auto" else SHAPES[shape])
        assert_layer_close(outs[shape], ref64, f"{cfg.name}/{shape}")
    # the tile shape only regroups rows: every output bit is the same
    first = outs[shapes[0]]
    for shape in shapes[1:]:
        assert np.array_equal(outs[shape], first), f"{cfg.name}: {shape} differs from {shapes[0]}"
    return first, ref_bits


def test_toy_config():
    _check_small(CONFIGS[0])


def test_tiny_k2_with_shared_expert():
    _check_small(Config("tiny_k2", 32, 256, 384, 16, 4, "rmsnorm", "uniform", "uniform", True, seed=11))


def test_shared_expert_stream_matches_one_stream():
    """moe_layer runs the shared expert on a second stream; the result must be bit-identical to
    the same calls made one after another on one stream (dispatch, routed experts, shared
    expert, combine), at every tile height, and stay so when the caller's stream is not the
    default one."""
    cfg = Config("side_stream", 300, 256, 384, 6, 3, "rmsnorm", "uniform", "uniform", True, seed=31)
    x_bits = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    exd = experts_dev(make_experts_host(cfg))
    shd = experts_dev(make_shared_host(cfg))
    x = bf16_dev(x_bits)
    t_ids = torch.from_numpy(ids).cuda()
    t_w = torch.from_numpy(w).cuda()
    for shape in ("auto", "16", "128", "224"):
        flags = 0 if shape == "auto" else SHAPES[shape]
        say(f"shared expert on a second stream, shape={shape}")
        disp = moe.dispatch(t_ids, cfg.E)
        y = moe.grouped_swiglu(x, disp, exd, flags)
        sh = moe.grouped_swiglu(x, moe.identity_dispatch(cfg.N, x.device), shd)
        one = bits_host(moe.combine(y, disp, t_w, sh))
        two = bits_host(moe.moe_layer(x, t_ids, t_w, exd, shd, flags=flags))
        torch.cuda.synchronize()
        assert np.array_equal(one, two), f"shape {shape}: two-stream result differs"
        caller = torch.cuda.Stream()
        caller.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(caller):
            three = moe.moe_layer(x, t_ids, t_w, exd, shd, flags=flags)
        torch.cuda.current_stream().wait_stream(caller)
        torch.cuda.synchronize()
        assert np.array_equal(bits_host(three), one), f"shape {shape}: result on a caller stream differs"


def test_ragged_dims():
    # d = 384: the down kernel's last 256-column block is half empty; 77 tokens: ragged tiles.
    # d_ff = 1024 keeps enough requantisation groups per row that the matrix cores' own
    # accumulation rounding (which flips ~0.15% of the e4m3 codes of h by one step) averages
    # out the way it does at the real d_ff = 2048.
    _check_small(Config("ragged", 77, 384, 1024, 5, 3, "normal", "uniform", "dirichlet", False, seed=3))


def test_skew_multiple_row_tiles():
    # 300 tokens all routed to experts 0 and 1: 300 rows per expert, several tiles in every shape
    cfg = Config("skew", 300, 256, 1024, 4, 2, "normal", "uniform", "uniform", True, seed=4)
    ids = np.tile(np.array([[1, 0]], np.int32), (300, 1))
    _, w = make_routing(cfg)
    _check_small(cfg, ids, w)


@pytest.mark.parametrize("K", [1, 2])
def test_expert_rows_at_tile_boundaries(K):
    # experts holding exactly one tile of each height, and one row more (a last tile of one
    # row): every tile edge of the 16-, 128-, 192- and 224-row kernels. K = 2: the gate|up
    # gather and the combine see every edge; K = 1: the down epilogue's top-1 combine does.
    counts = np.array([16, 17, 128, 129, 192, 193, 224, 225])
    E = len(counts)
    N = int(counts.sum()) // K
    cfg = Config(f"tile_edges_k{K}", N, 256, 256, E, K, "normal", "uniform", "dirichlet", False, seed=51)
    slots = np.repeat(np.arange(E, dtype=np.int32), counts)       # expert of each slot
    rng = np.random.default_rng(52)
    # token t takes slots t, t + N, ... of the slots sorted by expert: its experts differ,
    # since no expert holds more than N slots
    assert counts.max() <= N
    ids = np.stack([slots[k * N:(k + 1) * N] for k in range(K)], axis=1)
    assert K == 1 or np.all(ids[:, 0] != ids[:, 1])
    ids = ids[rng.permutation(N)]
    w = rng.dirichlet(np.ones(K), size=N).astype(np.float32)
    assert np.array_equal(np.bincount(ids.reshape(-1), minlength=E), counts)
    _check_small(cfg, ids, w)


def test_many_choices_per_token():
    # K = 12 > 8: the combine's second batch of source rows, part-filled; d = 1536: the second
    # 1024-column slice of a token covers only half a wave; with the shared expert
    _check_small(Config("k12", 40, 1536, 1024, 16, 12, "rmsnorm", "uniform", "dirichlet", True, seed=12))


def test_empty_experts_and_single_token():
    cfg = Config("sparse", 4, 256, 1024, 64, 2, "normal", "uniform", "uniform", False, seed=5)
    _check_small(cfg)
    cfg1 = Config("one_token", 1, 256, 1024, 8, 8, "rmsnorm", "uniform", "uniform", True, seed=6)
    _check_small(cfg1)


def test_zero_tokens():
    cfg = Config("empty", 0, 256, 128, 8, 2, "normal", "uniform", "uniform", False)
    exd = experts_dev(make_experts_host(cfg))
    say("layer N=0")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    out = moe.moe_layer(x, torch.empty((0, 2), dtype=torch.int32, device="cuda"),
                        torch.empty((0, 2), dtype=torch.float32, device="cuda"), exd)
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


def test_zero_input_gives_zero_output():
    cfg = CONFIGS[0]
    ids, w = make_routing(cfg)
    exd = experts_dev(make_experts_host(cfg))
    say("layer zero input")
    out = _layer(np.zeros((cfg.N, cfg.d), np.uint16), ids, w, exd)
    assert np.all(oracle.bf16_to_f32(out) == 0.0)


# --------------------------------------------------------------------------- size limits
def test_non_finite_inputs_give_nan_tokens_only():
    # x holds a NaN, a +inf and a -inf in three tokens. The quantiser's reading: an infinite
    # amax makes the group's scale infinite, x/s is then NaN for the infinite element, and a
    # NaN is encoded as the NaN code. So those tokens' outputs are NaN in every element, as
    # the oracle's are; every other token is untouched and within the layer tolerance, and
    # identical at every tile height.
    cfg = Config("nonfinite", 40, 384, 256, 6, 2, "normal", "uniform", "dirichlet", False, seed=41)
    x = make_x_bits(cfg).copy()
    x[3, 5] = 0x7FC0     # NaN
    x[7, 200] = 0x7F80   # +inf
    x[11, 0] = 0xFF80    # -inf
    ids, w = make_routing(cfg)
    exh = make_experts_host(cfg)
    _, ref64 = oracle.moe_forward(x, ids, w, exh)
    bad = np.array([3, 7, 11])
    good = np.setdiff1d(np.arange(cfg.N), bad)
    assert np.isnan(ref64[bad]).all() and np.isfinite(ref64[good]).all()
    exd = experts_dev(exh)
    first = None
    for shape in ("auto", "16", "128", "192", "224", "256"):
        say(f"layer nonfinite shape={shape}")
        out = _layer(x, ids, w, exd, None, 0 if shape == "auto" else SHAPES[shape])
        assert np.isnan(oracle.bf16_to_f32(out[bad])).all(), f"nonfinite/{shape}: a poisoned token is not all NaN"
        assert_layer_close(out[good], ref64[good], f"nonfinite/{shape}")
        if first is None:
            first = out[good]
        else:
            assert np.array_equal(out[good], first), f"nonfinite: {shape} differs on the finite tokens"


def test_maximum_hidden_size():
    # d = 65536 = MOE_MAX_DIM: 512 K blocks per gate|up row, which exactly fills the many-row
    # kernels' table of weight block scales; every tile height, against the oracle
    _check_small(Config("max_d", 48, 65536, 256, 4, 2, "normal", "uniform", "softmax", False, seed=31))


def test_activation_offsets_beyond_32_bits():
    """N * d >= 2^32: the many-row kernels' 32-bit activation offsets would overflow, so every
    tile height must fall back to the 16-row kernel (64-bit addressing). Rows past 2^32 bytes of
    x, x_q and y_sorted are compared with the oracle."""
    d, d_ff, E, K = 65536, 128, 2, 1
    N = 65536 + 16                         # x_q row 65536 starts at byte 2^32
    cfg = Config("offsets64", N, d, d_ff, E, K, "normal", "uniform", "uniform", False, seed=32)
    exh = make_experts_host(cfg)
    exd = experts_dev(exh)
    ids, w = make_routing(cfg)
    say("offsets64 inputs")
    gen = torch.Generator(device="cuda").manual_seed(32)
    x = torch.empty((N, d), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, N, 4096):          # drawn in chunks: float32 staging of the whole x is 17 GB
        r1 = min(N, r0 + 4096)
        x[r0:r1] = torch.randn((r1 - r0, d), generator=gen, device="cuda").to(torch.bfloat16)
    t_ids = torch.from_numpy(ids).cuda()
    t_w = torch.from_numpy(w).cuda()
    tok = np.array([0, 32767, 32768, 40000, 65535, 65536, N - 1], np.int64)
    outs = []
    for flags in (0, moe.FLAG_TILE_192):
        say(f"offsets64 layer flags={flags}")
        out = moe.moe_layer(x, t_ids, t_w, exd, flags=flags)
        torch.cuda.synchronize()
        outs.append(bits_host(out[torch.from_numpy(tok).cuda()]))
        del out
    assert np.array_equal(outs[0], outs[1])
    x_tok = bits_host(x[torch.from_numpy(tok).cuda()])
    del x
    say(f"offsets64 oracle tokens={len(tok)}")
    _, ref64 = oracle.moe_forward(x_tok, ids[tok], w[tok], exh)
    assert_layer_close(outs[0], ref64, "offsets64 sampled")


def test_profiler_times_only_the_selected_kinds():
    """moe_profile_enable_kinds: with only gate|up selected, a layer call records one gate|up
    launch and nothing for the other kinds; with every kind selected, each kind is counted."""
    cfg = CONFIGS[0]
    x = bf16_dev(make_x_bits(cfg))
    ids, w = make_routing(cfg)
    exd = experts_dev(make_experts_host(cfg))
    t_ids = torch.from_numpy(ids).cuda()
    t_w = torch.from_numpy(w).cuda()
    kinds = (moe.KERNEL_QUANT, moe.KERNEL_DISPATCH, moe.KERNEL_GATE_UP, moe.KERNEL_DOWN, moe.KERNEL_COMBINE)
    try:
        moe.profile_reset()
        moe.profile_enable(True, kinds=[moe.KERNEL_GATE_UP])
        moe.moe_layer(x, t_ids, t_w, exd)
        torch.cuda.synchronize()
        moe.profile_enable(False)
        counts = {k: moe.profile_read(k)[1] for k in kinds}
        assert counts[moe.KERNEL_GATE_UP] == 1
        assert all(counts[k] == 0 for k in kinds if k != moe.KERNEL_GATE_UP), counts
        moe.profile_reset()
        moe.profile_enable(True)
        moe.moe_layer(x, t_ids, t_w, exd)
        torch.cuda.synchronize()
        moe.profile_enable(False)
        counts = {k: moe.profile_read(k)[1] for k in kinds}
        assert all(counts[k] >= 1 for k in kinds), counts
        assert moe.profile_read(moe.KERNEL_GATE_UP)[0] > 0.0
    finally:
        moe.profile_enable(False)
        moe.profile_reset()

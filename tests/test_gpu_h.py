"""GPU: each expert's own results against the oracle's for every (token, expert) pair: the
requantised product h = e4m3(silu(g) * u) that the gate|up epilogue writes, code by code, and
the down projection's bf16 rows y_sorted, which the layer test sees only after the combine.

White-box: moe_grouped_swiglu_q's workspace holds h first (its quantised activations are the
caller's): the e4m3 codes [rows][d_ff] in sorted-position order at offset 0, then their
float32 scales [rows][d_ff/128] from the next 256-byte boundary.

With exact block sums the GPU's g and u differ from the oracle's float64 values only by
float32 rounding, so a code of h may move by one step where h/s lies within that rounding of
an e4m3 midpoint, and a group scale may differ by a few float32 ulps. Measured at K2 shapes:
45 of 4,194,304 codes moved (0.0011%), none by more than one step, scales within 1e-6. The
FP8 matrix ops' rounded sums moved about 0.15% of the codes, which this bar rejects."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
from mixture_experts_ffn_ids_amd import api
import oracle
from parity import bf16_dev, bits_host, experts_dev, say
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host

pytestmark = pytest.mark.gpu

MOVED_MAX = 1e-4        # share of h codes allowed to differ (one step each)
SCALE_REL_MAX = 1e-5    # relative difference of the group scales
# y_sorted, one expert's output row in bf16: measured at K2 dimensions, 97.5% of the values are
# the oracle's own bf16 rounding, each row's relative L2 error at most 2.6e-3 (median 1.66e-3,
# the bf16 rounding itself) and the largest error 3.3e-3 of the largest value. The rest comes
# from the moved codes of h and the FP8 matrix op's rounded sums in down.
Y_SAME_MIN = 0.95
Y_ROW_REL_MAX = 4e-3
Y_ELEM_MAX = 5e-3

CASES = [
    # several row tiles per expert at every height; d_ff = 512: four requantisation groups
    Config("h_small", 96, 512, 512, 6, 2, "normal", "uniform", "dirichlet", False, seed=81),
    # K2 dimensions, 16 experts: 2048 rows of d_ff = 2048 over d = 7168
    Config("h_k2", 256, 7168, 2048, 16, 8, "rmsnorm", "uniform", "dirichlet", False, seed=82),
]
TILES = [0, moe.FLAG_TILE_16, moe.FLAG_TILE_128, moe.FLAG_TILE_192, moe.FLAG_TILE_224, moe.FLAG_TILE_256]
TILE_IDS = ["auto", "16", "128", "192", "224", "256"]


def _gpu_h(xq, xs, disp, exd, flags, rows, d_ff):
    moe.grouped_swiglu_q(xq, xs, disp, exd, flags, _ws_tag="h_check")
    torch.cuda.synchronize()
    ws = api._WS_CACHE[(str(xq.device), torch.cuda.current_stream(xq.device).cuda_stream, "h_check")].cpu().numpy()
    hq = ws[:rows * d_ff].reshape(rows, d_ff).copy()
    off = (rows * d_ff + 255) // 256 * 256
    hs = ws[off:off + rows * (d_ff // 128) * 4].view(np.float32).reshape(rows, d_ff // 128).copy()
    return hq, hs


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_requantised_h_against_the_oracle(cfg):
    x = make_x_bits(cfg)
    ids, _ = make_routing(cfg)
    exh = make_experts_host(cfg)
    exd = experts_dev(exh)
    xq, xs = moe.quantize_rows(bf16_dev(x))
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), cfg.E)
    ss = disp.sorted_slot.cpu().numpy()
    rows = cfg.N * cfg.K
    # sorted position p holds slot ss[p]: token ss[p] // K through expert ids[token, ss[p] % K]
    _, hq_ref, hs_ref = oracle.expert_rows(x, exh, ss // cfg.K, ids.reshape(-1)[ss])
    values = np.unique(oracle.e4m3_decode(np.arange(256, dtype=np.uint8)))
    values = values[~np.isnan(values)]
    first = None
    for flags, name in zip(TILES, TILE_IDS):
        say(f"h {cfg.name} tile={name}")
        hq, hs = _gpu_h(xq, xs, disp, exd, flags, rows, cfg.d_ff)
        srel = np.abs(hs.astype(np.float64) / hs_ref.astype(np.float64) - 1.0).max()
        assert srel <= SCALE_REL_MAX, f"{cfg.name}/{name}: group scales differ by {srel:.3e} (relative)"
        gv, rv = oracle.e4m3_decode(hq), oracle.e4m3_decode(hq_ref)
        assert not np.isnan(gv).any() and not np.isnan(rv).any()
        moved = hq != hq_ref
        steps = np.abs(np.searchsorted(values, gv).astype(np.int64) - np.searchsorted(values, rv).astype(np.int64))
        print(f"[h] {cfg.name}/{name}: {moved.sum()} of {moved.size} codes moved, scales within {srel:.2e}",
              flush=True)
        assert steps.max() <= 1, f"{cfg.name}/{name}: a code moved by {steps.max()} steps"
        assert moved.mean() <= MOVED_MAX, f"{cfg.name}/{name}: {moved.mean():.3%} of the codes moved"
        # the tile height only regroups rows: h is the same bit for bit
        if first is None:
            first = (hq, hs)
        else:
            assert np.array_equal(hq, first[0]) and np.array_equal(hs.view(np.uint32), first[1].view(np.uint32))


@pytest.mark.parametrize("cfg", CASES, ids=[c.name for c in CASES])
def test_expert_output_rows_against_the_oracle(cfg):
    x = make_x_bits(cfg)
    ids, _ = make_routing(cfg)
    exh = make_experts_host(cfg)
    exd = experts_dev(exh)
    disp = moe.dispatch(torch.from_numpy(ids).cuda(), cfg.E)
    ss = disp.sorted_slot.cpu().numpy()
    y_ref, _, _ = oracle.expert_rows(x, exh, ss // cfg.K, ids.reshape(-1)[ss])
    ref_bf16 = oracle.bf16_to_f32(oracle.bf16_from_f64(y_ref)).astype(np.float64)
    x_d = bf16_dev(x)
    for flags, name in zip(TILES, TILE_IDS):
        say(f"y_sorted {cfg.name} tile={name}")
        y = bits_host(moe.grouped_swiglu(x_d, disp, exd, flags))
        torch.cuda.synchronize()
        g = oracle.bf16_to_f32(y).astype(np.float64)
        same = (g == ref_bf16).mean()
        rel = np.sqrt(((g - y_ref) ** 2).sum(axis=1)) / np.sqrt((y_ref ** 2).sum(axis=1))
        elem = np.abs(g - y_ref).max() / np.abs(y_ref).max()
        print(f"[y] {cfg.name}/{name}: {same:.2%} bf16-identical, row rel L2 <= {rel.max():.2e}, "
              f"elementwise <= {elem:.2e} of max", flush=True)
        assert same >= Y_SAME_MIN, f"{cfg.name}/{name}: only {same:.2%} of y_sorted matches the oracle's bf16"
        assert rel.max() <= Y_ROW_REL_MAX, f"{cfg.name}/{name}: a row's relative L2 error is {rel.max():.3e}"
        assert elem <= Y_ELEM_MAX, f"{cfg.name}/{name}: elementwise error {elem:.3e} of max"

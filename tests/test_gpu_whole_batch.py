"""GPU: every token of every full-size workload against the oracle, element by element, in the
launch configuration the benchmark times (automatic tile height).

For each workload:
  - dispatch (counts, offsets, sorted_slot, slot_pos) equals the oracle's bit for bit;
  - two runs give the same bits, and the 16-row tile kernel (FLAG_TILE_16) gives the same bits
    as the automatic choice on every row: the tile height only regroups rows, so the row-group
    sweep, the XCD item order and every tile edge are covered by the identity;
  - every output token is within the layer tolerance of the oracle (per-token relative L2 and
    the elementwise bar against the largest |ref| of the whole batch).
The oracle runs over the batch in chunks of tokens, printing its progress; the whole-batch
maxima are printed as one "[whole-batch]" line per workload and, when MOE_PARITY_RECORD names
a file, appended to it as JSON lines.
"""
import json
import os
import time

import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import WholeBatch, bf16_dev, bits_host, say
from workloads import config_by_name, make_routing, make_x_bits
from workloads.gen import experts_to_host, make_block_inputs, make_experts_device, make_shared_device

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

EPS = 1e-6
_HOST: dict = {}


def _host(exd):
    """Host copy of a device expert set, kept for the other tests of this module (the 16.9 GB
    routed set is shared by the four K2 layer workloads)."""
    key = id(exd)
    if key not in _HOST:
        t0 = time.perf_counter()
        _HOST[key] = (exd, experts_to_host(exd))
        say(f"host copy of {exd.E} experts (d_ff {exd.d_ff}) in {time.perf_counter() - t0:.1f} s")
    return _HOST[key][1]


def _record(what: str, summary: dict):
    path = os.environ.get("MOE_PARITY_RECORD")
    if path:
        with open(path, "a") as f:
            f.write(json.dumps({"case": what, **summary}) + "\n")


def _check_dispatch(ids, E):
    d = moe.dispatch(torch.from_numpy(ids).cuda(), E)
    c, o, ss, sp = oracle.dispatch(ids, E)
    assert np.array_equal(d.counts.cpu().numpy(), c) and np.array_equal(d.offsets.cpu().numpy(), o)
    assert np.array_equal(d.sorted_slot.cpu().numpy(), ss) and np.array_equal(d.slot_pos.cpu().numpy(), sp)


def _compare(what, out_bits, x_bits, ids, w, exh, shh=None, residual=None, chunk=1024):
    """The oracle over all tokens, chunk by chunk, against the GPU output."""
    N = out_bits.shape[0]
    wb = WholeBatch(what, N)
    t0 = time.perf_counter()
    for a in range(0, N, chunk):
        tok = np.arange(a, min(N, a + chunk), dtype=np.int64)
        if residual is None:
            _, ref64 = oracle.moe_forward(x_bits, ids, w, exh, shh, tokens=tok)
        else:
            _, ref64 = oracle.moe_forward(x_bits, ids, w, exh, shh, tokens=tok, residual=residual)
        wb.add(tok, out_bits[tok], ref64)
        print(f"[oracle] {what}: {tok[-1] + 1}/{N} tokens, {time.perf_counter() - t0:.1f} s", flush=True)
    s = wb.check()
    _record(what, s)


def _layer(x, t_ids, t_w, exd, shd, flags):
    out = moe.moe_layer(x, t_ids, t_w, exd, shd, flags=flags)
    torch.cuda.synchronize()
    return bits_host(out)


@pytest.mark.parametrize("name", ["k2_decode_16", "k2_decode_256", "k2_prefill_8192", "k2_skewed_shared_4096",
                                  "k2_ep8_shard_8192"])
def test_whole_batch(name):
    cfg = config_by_name(name)
    x_bits = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    say(f"whole batch {name}: weights")
    exd = make_experts_device(cfg)
    shd = make_shared_device(cfg) if cfg.shared else None
    x, t_ids, t_w = bf16_dev(x_bits), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda()
    say(f"whole batch {name}: layer")
    out = _layer(x, t_ids, t_w, exd, shd, 0)
    assert np.array_equal(out, _layer(x, t_ids, t_w, exd, shd, 0)), "two runs differ"
    say(f"whole batch {name}: 16-row tiles")
    assert np.array_equal(out, _layer(x, t_ids, t_w, exd, shd, moe.FLAG_TILE_16)), \
        "automatic tile height and 16-row tiles differ"
    del x, t_ids, t_w
    _check_dispatch(ids, cfg.E)
    exh = _host(exd)
    shh = experts_to_host(shd) if shd is not None else None
    _compare(name, out, x_bits, ids, w, exh, shh)


def test_whole_batch_prefill_block():
    """hidden + layer(RMSNorm(hidden)) at the 8192-token prefill shapes, every token."""
    cfg = config_by_name("k2_prefill_8192")
    h_bits, g_bits = make_block_inputs(cfg)
    ids, w = make_routing(cfg)
    say("whole batch prefill block: weights")
    exd = make_experts_device(cfg)
    args = (bf16_dev(g_bits), EPS, torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda(), exd)
    say("whole batch prefill block: layer")
    out = bits_host(moe.moe_block_ffn(bf16_dev(h_bits), *args))
    say("whole batch prefill block: 16-row tiles")
    out16 = bits_host(moe.moe_block_ffn(bf16_dev(h_bits), *args, flags=moe.FLAG_TILE_16))
    torch.cuda.synchronize()
    assert np.array_equal(out, out16), "automatic tile height and 16-row tiles differ"
    exh = _host(exd)
    x_norm = oracle.rmsnorm_rows(h_bits, g_bits, EPS)
    _compare("k2_prefill_8192 block", out, x_norm, ids, w, exh, residual=h_bits)


def test_whole_batch_dense():
    """The dense block's MLP (8192 tokens, d_ff 18432), every token."""
    cfg = config_by_name("k2_dense_8192")
    x_bits = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    say("whole batch dense: weights")
    exd = make_experts_device(cfg)
    x = bf16_dev(x_bits)
    say("whole batch dense: mlp")
    out = bits_host(moe.dense_swiglu(x, exd))
    assert np.array_equal(out, bits_host(moe.dense_swiglu(x, exd))), "two runs differ"
    say("whole batch dense: 16-row tiles")
    assert np.array_equal(out, bits_host(moe.dense_swiglu(x, exd, flags=moe.FLAG_TILE_16))), \
        "automatic tile height and 16-row tiles differ"
    exh = _host(exd)
    _compare("k2_dense_8192", out, x_bits, ids, w, exh, chunk=512)

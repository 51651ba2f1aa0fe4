"""GPU: moe_dispatch must equal the oracle's dispatch bit for bit (counts, offsets, the
stable order of slots and its inverse) on every workload and on the edge cases."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import say
from workloads import CONFIGS, make_routing

pytestmark = pytest.mark.gpu


def _run(ids: np.ndarray, E: int, checked=False):
    t = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int32)).cuda()
    d = moe.dispatch(t, E, checked=checked)
    torch.cuda.synchronize()
    return d


def _assert_same(ids, E):
    say(f"dispatch N={ids.shape[0]} K={ids.shape[1]} E={E}")
    d = _run(ids, E)
    c, o, ss, sp = oracle.dispatch(ids, E)
    assert np.array_equal(d.counts.cpu().numpy(), c)
    assert np.array_equal(d.offsets.cpu().numpy(), o)
    assert np.array_equal(d.sorted_slot.cpu().numpy(), ss)
    assert np.array_equal(d.slot_pos.cpu().numpy(), sp)
    return d


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_dispatch_configs_bit_exact(cfg):
    ids, _ = make_routing(cfg)
    _assert_same(ids, cfg.E)


def test_dispatch_edge_cases():
    rng = np.random.default_rng(0)
    _assert_same(np.zeros((1, 1), np.int32), 1)                                 # N = 1, K = 1, E = 1
    _assert_same(np.zeros((777, 1), np.int32), 1)                               # identity dispatch, ragged chunks
    _assert_same(np.tile(np.arange(8, dtype=np.int32), (33, 1)), 8)             # K = E
    _assert_same(np.tile(np.array([[5, 2]], np.int32), (1000, 1)), 16)          # all tokens to two experts
    _assert_same(np.argsort(rng.random((3, 8192)), 1)[:, :8].astype(np.int32), 8192)   # E at the limit
    _assert_same(np.argsort(rng.random((5000, 64)), 1)[:, :8].astype(np.int32), 64)    # many chunks
    _assert_same(np.argsort(rng.random((31, 64)), 1)[:, :64].astype(np.int32), 64)     # K = 64 (limit)
    _assert_same(np.argsort(rng.random((333, 5)), 1).astype(np.int32), 5)              # E not a multiple of 4,
    _assert_same(np.argsort(rng.random((4999, 7)), 1)[:, :3].astype(np.int32), 7)     # ragged last chunk


def test_dispatch_empty():
    say("dispatch N=0")
    d = _run(np.zeros((0, 4), np.int32), 8)
    assert np.all(d.counts.cpu().numpy() == 0) and np.all(d.offsets.cpu().numpy() == 0)


def test_dispatch_checked_mode():
    ids = np.array([[0, 3], [1, 2]], np.int32)
    say("dispatch checked ok")
    _run(ids, 4, checked=True)
    bad = np.array([[0, 4], [1, 2]], np.int32)
    say("dispatch checked bad id")
    with pytest.raises(moe.MoeError) as ei:
        _run(bad, 4, checked=True)
    assert ei.value.status == 5
    neg = np.array([[0, -1]], np.int32)
    with pytest.raises(moe.MoeError) as ei:
        _run(neg, 4, checked=True)
    assert ei.value.status == 5
    dup = np.array([[0, 1], [2, 2]], np.int32)
    say("dispatch checked duplicate id")
    with pytest.raises(moe.MoeError) as ei:
        _run(dup, 4, checked=True)
    assert ei.value.status == 6


def test_dispatch_unchecked_bad_ids_are_memory_safe():
    """Without checking, out-of-range slots are left out (slot_pos = -1)."""
    ids = np.array([[0, 9], [1, 2]], np.int32)
    say("dispatch unchecked bad id")
    d = _run(ids, 4)
    sp = d.slot_pos.cpu().numpy()
    assert sp[1] == -1
    assert d.counts.cpu().numpy().sum() == 3


def test_dispatch_deterministic():
    cfg = CONFIGS[3]
    ids, _ = make_routing(cfg)
    say("dispatch determinism")
    a = _run(ids, cfg.E)
    b = _run(ids, cfg.E)
    for x, y in ((a.counts, b.counts), (a.offsets, b.offsets), (a.sorted_slot, b.sorted_slot),
                 (a.slot_pos, b.slot_pos)):
        assert torch.equal(x, y)

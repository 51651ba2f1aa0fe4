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


@pytest.mark.parametrize("n, k, E", [(1024, 8, 384), (1025, 8, 384), (2, 1, 4096), (2, 1, 4097),
                                     (1000, 8, 4096), (8191, 1, 3)],
                         ids=["8192-slots", "8200-slots", "E4096", "E4097", "8000-slots-E4096", "8191-slots-E3"])
def test_dispatch_at_the_one_workgroup_limits(n, k, E):
    """Batches of at most 8192 slots and 4096 experts take the one-workgroup dispatch, larger
    ones the four-launch path; both must give the oracle's result on either side of the limits."""
    rng = np.random.default_rng(n * 31 + E)
    ids = np.argsort(rng.random((n, E)), 1)[:, :k].astype(np.int32) if E <= 512 else \
        np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    _assert_same(ids, E)


@pytest.mark.parametrize("n", [7, 1500], ids=["one-wave", "two-rounds"])
def test_dispatch_unchecked_bad_ids_small_batch(n):
    """The one-workgroup dispatch leaves out-of-range slots out like the four-launch path:
    counts of the valid ids only, valid slots in stable order, slot_pos = -1 for the rest
    (compared with numpy's bincount and stable argsort)."""
    E = 6
    rng = np.random.default_rng(n)
    ids = rng.integers(-2, E + 2, size=(n, 2)).astype(np.int32)
    say(f"dispatch unchecked bad ids N={n}")
    d = _run(ids, E)
    flat = ids.ravel()
    valid = (flat >= 0) & (flat < E)
    order = np.nonzero(valid)[0][np.argsort(flat[valid], kind="stable")]
    pos = np.full(flat.size, -1, np.int64)
    pos[order] = np.arange(order.size)
    assert np.array_equal(d.counts.cpu().numpy(), np.bincount(flat[valid], minlength=E))
    assert np.array_equal(d.sorted_slot.cpu().numpy()[:order.size], order)
    assert np.array_equal(d.slot_pos.cpu().numpy(), pos)

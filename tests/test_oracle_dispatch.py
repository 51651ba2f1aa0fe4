"""Pins of the oracle's dispatch (histogram, prefix sum, stable permutation).

The "Mixture of experts" page (experts inspector, Code: moe_infer) counts the
tokens per expert with a scatter of ones and a column sum, orders the flat
slots by expert with an argsort, runs each expert on its contiguous slice
(running start/end indices) and scatters outputs back with the inverse order.
The tie order of that argsort is unspecified on the page; the oracle fixes it
to ascending slot index, so it must equal numpy's stable argsort.
"""
import numpy as np
import pytest

import oracle
from workloads import CONFIGS, make_routing


def _check_dispatch(ids, E):
    N, K = ids.shape
    counts, offsets, sorted_slot, slot_pos = oracle.dispatch(ids, E)
    flat = ids.ravel()
    # histogram: library bincount, sums to N*K
    assert np.array_equal(counts, np.bincount(flat, minlength=E).astype(np.int32))
    assert counts.sum() == N * K
    # prefix sum
    assert offsets[0] == 0 and np.array_equal(offsets[1:], np.cumsum(counts))
    # permutation of [0, NK), equal to the stable argsort, sorted keys, slices per expert
    assert np.array_equal(np.sort(sorted_slot), np.arange(N * K))
    assert np.array_equal(sorted_slot, np.argsort(flat, kind="stable").astype(np.int32))
    keys = flat[sorted_slot]
    assert np.all(np.diff(keys) >= 0)
    for e in range(E):
        assert np.all(keys[offsets[e]:offsets[e + 1]] == e)
        # empty expert <=> empty slice
        assert (offsets[e] == offsets[e + 1]) == (counts[e] == 0)
    # inverse
    assert np.array_equal(slot_pos[sorted_slot], np.arange(N * K))
    assert np.array_equal(sorted_slot[slot_pos], np.arange(N * K))
    return counts, offsets, sorted_slot, slot_pos


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_dispatch_configs(cfg):
    ids, _ = make_routing(cfg)
    counts, *_ = _check_dispatch(ids, cfg.E)
    if cfg.name == "k2_decode_16":
        assert (counts == 0).sum() > 200          # most experts untouched at 16 tokens


def test_dispatch_brute_force_tiny():
    """Every ids matrix over E=3, N=2, K=2 with distinct ids per row, by enumeration."""
    rows = [(a, b) for a in range(3) for b in range(3) if a != b]
    for r0 in rows:
        for r1 in rows:
            ids = np.array([r0, r1], np.int32)
            counts, offsets, sorted_slot, slot_pos = oracle.dispatch(ids, 3)
            # brute force: positions listed expert by expert, slots in increasing order
            order = [s for e in range(3) for s in range(4) if ids.ravel()[s] == e]
            assert list(sorted_slot) == order
            assert [list(ids.ravel()).count(e) for e in range(3)] == list(counts)


def test_dispatch_edge_cases():
    _check_dispatch(np.zeros((0, 4), np.int32), 8)                 # no tokens
    _check_dispatch(np.array([[3]], np.int32), 8)                   # one token, K = 1
    _check_dispatch(np.zeros((50, 1), np.int32), 1)                 # E = 1 identity dispatch
    ids = np.tile(np.arange(8, dtype=np.int32), (5, 1))             # K = E
    _check_dispatch(ids, 8)
    ids = np.tile(np.array([[7, 2]], np.int32), (33, 1))            # all tokens to the same two experts
    counts, *_ = _check_dispatch(ids, 16)
    assert counts[7] == 33 and counts[2] == 33 and counts.sum() == 66
    # identity dispatch is the identity permutation
    _, offsets, sorted_slot, slot_pos = oracle.dispatch(np.zeros((9, 1), np.int32), 1)
    assert list(offsets) == [0, 9] and list(sorted_slot) == list(range(9)) == list(slot_pos)


def test_dispatch_rejects_bad_and_duplicate_ids():
    with pytest.raises(oracle.OracleError, match="bad expert id"):
        oracle.dispatch(np.array([[0, 8]], np.int32), 8)
    with pytest.raises(oracle.OracleError, match="bad expert id"):
        oracle.dispatch(np.array([[-1, 2]], np.int32), 8)
    with pytest.raises(oracle.OracleError, match="duplicate"):
        oracle.dispatch(np.array([[1, 2], [3, 3]], np.int32), 8)
    with pytest.raises(oracle.OracleError, match="shape"):
        oracle.dispatch(np.zeros((2, 9), np.int32), 8)              # K > E

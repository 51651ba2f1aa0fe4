"""The seeded input generators are deterministic: the same seed gives the same bytes, a
different seed different ones (they feed both the oracle and the GPU path)."""
import numpy as np

from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_block_inputs, make_experts_host, make_shared_host

CFG = Config("gen", 40, 256, 128, 8, 3, "rmsnorm", "uniform", "softmax", True, seed=3)
ZIPF = Config("genz", 60, 256, 128, 16, 4, "normal", "zipf", "dirichlet", False, seed=4)


def _all(cfg, seed=None):
    x = make_x_bits(cfg, seed)
    ids, w = make_routing(cfg, seed)
    h, g = make_block_inputs(cfg, seed)
    ex = make_experts_host(cfg, seed)
    out = [x, ids, w, h, g, ex.w_gate, ex.s_gate, ex.w_up, ex.s_up, ex.w_down, ex.s_down]
    if cfg.shared:
        sh = make_shared_host(cfg, seed)
        out += [sh.w_gate, sh.s_down]
    return out


def test_same_seed_same_bytes():
    for cfg in (CFG, ZIPF):
        a, b = _all(cfg), _all(cfg)
        for u, v in zip(a, b):
            assert u.dtype == v.dtype and u.shape == v.shape
            assert u.tobytes() == v.tobytes()


def test_other_seed_other_bytes():
    a, b = _all(CFG), _all(CFG, seed=CFG.seed + 1)
    # every random array changes (the gain is the constant 1 by recipe)
    for i, (u, v) in enumerate(zip(a, b)):
        if i == 4:
            assert np.all(u == 0x3F80) and np.all(v == 0x3F80)
        else:
            assert u.tobytes() != v.tobytes(), i


def test_routing_rows_are_distinct_and_weights_normalised():
    for cfg in (CFG, ZIPF):
        ids, w = make_routing(cfg)
        assert ids.dtype == np.int32 and ids.min() >= 0 and ids.max() < cfg.E
        assert all(len(set(r)) == cfg.K for r in ids.tolist())
        assert np.allclose(w.sum(1), 1.0, atol=1e-6) and np.all(w >= 0)

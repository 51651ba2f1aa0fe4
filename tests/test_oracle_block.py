"""Pins of the oracle's two block steps around the layer: the post-attention RMSNorm and the
second residual addition ("Input features" page, evidences "rmsnorm" and "block").

RMSNorm is pinned to closed forms and exact invariances rather than to its own formula:
  * one nonzero entry in a row of n: the mean of squares is v^2 / n, so the normalised entry
    is sign(v) sqrt(n) -- exactly 16 for n = 256 -- and every other entry is 0;
  * scaling a row by a power of two changes nothing when eps = 0;
  * a constant row normalises to +-1;
  * a zero row stays zero (eps keeps the reciprocal finite);
  * against the real-number value g x / sqrt(mean x^2 + eps), within the two bf16 roundings;
  * the intermediate bf16 rounding before the gain (the input dtype the page returns to) is
    visible on a row whose normalised entry is sqrt(128), not a bf16 number.
The residual addition: zero routing weights give the residual back exactly, and the residual
shifts the unrounded output by exactly its own value."""
import numpy as np
import pytest

import oracle
from workloads import Config, make_routing, make_x_bits
from workloads.gen import make_experts_host


def bf16_bits(v) -> np.ndarray:
    return oracle.bf16_from_f64(np.asarray(v, np.float64))


def f(bits) -> np.ndarray:
    return oracle.bf16_to_f32(np.asarray(bits, np.uint16)).astype(np.float64)


# |v| within float32's range for v^2 (the page squares in float32)
@pytest.mark.parametrize("v,g", [(3.0, 1.5), (-0.0078125, 1.0), (1e15, 0.25), (-3e-15, 2.0)])
def test_single_nonzero_entry_normalises_to_sqrt_n(v, g):
    n = 256
    x = np.zeros((1, n))
    x[0, 37] = v
    gain = np.full(n, g)
    y = f(oracle.rmsnorm_rows(bf16_bits(x), bf16_bits(gain), 0.0))
    expect = np.zeros((1, n))
    expect[0, 37] = np.sign(f(bf16_bits(v))) * 16.0 * g
    assert np.array_equal(y, expect)


def test_intermediate_rounding_to_the_input_dtype():
    # n = 128, one entry 1: the normalised entry is sqrt(128) = 11.3137..., which bf16 holds as
    # 11.3125. The page returns to the input dtype before the gain, so y = bf16(g * 11.3125).
    # For these gains that differs from rounding g * sqrt(128) once.
    n = 128
    x = np.zeros((1, n))
    x[0, 5] = 1.0
    for gv, two_roundings, one_rounding in ((1.046875, 11.8125, 11.875), (1.2734375, 14.375, 14.4375),
                                            (1.7734375, 20.0, 20.125)):
        y = f(oracle.rmsnorm_rows(bf16_bits(x), bf16_bits(np.full(n, gv)), 0.0))
        assert y[0, 5] == two_roundings != one_rounding
        assert np.count_nonzero(y) == 1


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 384))
    gain = rng.uniform(0.5, 2.0, 384)
    y0 = oracle.rmsnorm_rows(bf16_bits(x), bf16_bits(gain), 0.0)
    for k in (-40, -3, 5, 60):
        yk = oracle.rmsnorm_rows(bf16_bits(x * 2.0 ** k), bf16_bits(gain), 0.0)
        assert np.array_equal(yk, y0), k


def test_constant_and_zero_rows():
    n = 512
    x = np.stack([np.full(n, 0.3), np.full(n, -7.0), np.zeros(n)])
    y = f(oracle.rmsnorm_rows(bf16_bits(x), bf16_bits(np.ones(n)), 0.0 + 1e-6))
    assert np.all(y[0] == 1.0) and np.all(y[1] == -1.0)
    assert np.all(y[2] == 0.0) and np.all(np.isfinite(y))


def test_close_to_the_real_number_value():
    rng = np.random.default_rng(6)
    n = 7168
    x = f(bf16_bits(rng.standard_normal((5, n)) * rng.uniform(0.01, 100.0, (5, 1))))
    gain = f(bf16_bits(rng.uniform(0.1, 3.0, n)))
    eps = 1e-6
    y = f(oracle.rmsnorm_rows(bf16_bits(x), bf16_bits(gain), eps))
    ref = gain * x / np.sqrt((x ** 2).mean(axis=1, keepdims=True) + np.float32(eps))
    # two bf16 roundings (at most 2^-8 relative each: 8 significant bits) and float32 steps
    assert np.all(np.abs(y - ref) <= np.abs(ref) * (2 * 2.0 ** -8 + 2.0 ** -20) + 1e-30)


def _tiny():
    cfg = Config("tiny_res", 24, 256, 128, 6, 2, "normal", "uniform", "softmax", True, seed=41)
    ids, w = make_routing(cfg)
    return cfg, make_x_bits(cfg), ids, w, make_experts_host(cfg)


def test_zero_weights_return_the_residual():
    cfg, x, ids, w, ex = _tiny()
    res = bf16_bits(np.random.default_rng(7).standard_normal((cfg.N, cfg.d)) * 3.0)
    out, _ = oracle.moe_forward(x, ids, np.zeros_like(w), ex, residual=res)
    assert np.array_equal(out, res)


def test_residual_shifts_the_unrounded_output_by_itself():
    cfg, x, ids, w, ex = _tiny()
    res = bf16_bits(np.random.default_rng(8).standard_normal((cfg.N, cfg.d)))
    _, base = oracle.moe_forward(x, ids, w, ex)
    _, with_res = oracle.moe_forward(x, ids, w, ex, residual=res)
    diff = with_res - base
    assert np.allclose(diff, f(res), rtol=0, atol=1e-12 * np.abs(base).max() + 1e-300)

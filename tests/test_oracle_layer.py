"""Pins of the oracle's layer output against what the pages and mathematics fix.

* parameter counts printed on the "Mixture of experts" page (golden fixture);
* a dense all-experts-masked evaluation written with torch library routines
  (F.linear, F.silu, the float8_e4m3fn cast): out = sum_e G[n,e] E_e(x_n), with
  G the dense routing matrix -- a different formulation of the same sum, which
  with E = 1, K = 1, w = 1 is exactly the expert MLP forward of the "SwiGLU
  output" page (evidence "mlp": down(act(gate x) * up x));
* a closed form: permutation weight matrices make every term of the expert
  computable by hand;
* algebraic invariants of the weighted combine and the shared expert add
  ("Mixture of experts" page, Code: moe_infer weighted sum and forward's shared
  expert add).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from workloads import CONFIGS, Config, make_routing, make_x_bits
from workloads.gen import HostExperts, make_experts_host, make_shared_host

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                vals[k] = int(v)
    return vals


def test_parameter_counts_match_page():
    g = _read_golden("param_counts.txt")
    shapes = oracle.expert_weight_shapes(g["hidden_size"], g["moe_intermediate_size"])
    counts = {k: math.prod(v) for k, v in shapes.items()}
    assert counts["gate"] == g["gate_proj"]
    assert counts["up"] == g["up_proj"]
    assert counts["down"] == g["down_proj"]
    assert sum(counts.values()) == g["per_expert"]
    assert sum(counts.values()) * g["moe_blocks"] * g["routed_experts"] == g["all_routed"]
    # the scales are metadata outside the count: 2,688 per expert at K2 shapes
    sc = oracle.expert_scale_shapes(g["hidden_size"], g["moe_intermediate_size"])
    assert sum(math.prod(v) for v in sc.values()) == 2688


# --------------------------------------------------------------------------- dense reference
def _torch_quant(v: torch.Tensor) -> torch.Tensor:
    """Dequantised per-128-group e4m3 values of float32 rows, with torch's codec."""
    r, c = v.shape
    g = v.reshape(r, c // 128, 128)
    amax = g.abs().amax(-1, keepdim=True)
    s = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (g / s).to(torch.float8_e4m3fn).to(torch.float64)
    return (q * s.to(torch.float64)).reshape(r, c)


def _dequant_w(codes: np.ndarray, scales: np.ndarray) -> torch.Tensor:
    q = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    s = torch.from_numpy(scales).to(torch.float64)
    s = s.repeat_interleave(128, 0).repeat_interleave(128, 1)
    return q * s


def _mlp(xt: torch.Tensor, ex: HostExperts, e: int) -> torch.Tensor:
    """down(silu(gate x) * up x) with FP8 weights and the two activation quantisation points."""
    g = F.linear(xt, _dequant_w(ex.w_gate[e], ex.s_gate[e]))
    u = F.linear(xt, _dequant_w(ex.w_up[e], ex.s_up[e]))
    h = (F.silu(g) * u).to(torch.float32)
    return F.linear(_torch_quant(h), _dequant_w(ex.w_down[e], ex.s_down[e]))


def dense_reference(x_bits, ids, w, ex: HostExperts, shared: HostExperts | None = None):
    N = x_bits.shape[0]
    xf = torch.from_numpy(oracle.bf16_to_f32(x_bits).copy())
    xt = _torch_quant(xf)
    G = torch.zeros((N, ex.E), dtype=torch.float64)
    G.scatter_(1, torch.from_numpy(ids.astype(np.int64)), torch.from_numpy(w.astype(np.float64)))
    acc = torch.zeros((N, ex.d), dtype=torch.float64)
    for e in range(ex.E):                     # every expert on every token, masked by G
        acc += G[:, e:e + 1] * _mlp(xt, ex, e)
    if shared is not None:
        acc += _mlp(xt, shared, 0)
    return acc.numpy()


def _compare(out64, ref, bits=None, tol=1e-9):
    scale = np.abs(ref).max()
    assert np.abs(out64 - ref).max() <= tol * scale
    if bits is not None:
        ref_bits = oracle.bf16_from_f64(ref)
        assert (bits != ref_bits).mean() < 1e-3


TINY = Config("tiny_k2", 32, 256, 384, 16, 4, "rmsnorm", "uniform", "uniform", True, seed=11)


@pytest.mark.parametrize("cfg", [CONFIGS[0], TINY], ids=["toy", "tiny_k2"])
def test_oracle_matches_dense_masked_reference(cfg):
    x = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    ex = make_experts_host(cfg)
    sh = make_shared_host(cfg) if cfg.shared else None
    bits, out64 = oracle.moe_forward(x, ids, w, ex, sh)
    ref = dense_reference(x, ids, w, ex, sh)
    _compare(out64, ref, bits)


def test_single_expert_is_the_mlp_forward():
    """E = 1, K = 1, w = 1: the layer reduces to one expert MLP on every token."""
    cfg = Config("one", 16, 256, 256, 1, 1, "normal", "uniform", "uniform", False, seed=2)
    x = make_x_bits(cfg)
    ex = make_experts_host(cfg)
    ids = np.zeros((16, 1), np.int32)
    w = np.ones((16, 1), np.float32)
    bits, out64 = oracle.moe_forward(x, ids, w, ex)
    xt = _torch_quant(torch.from_numpy(oracle.bf16_to_f32(x).copy()))
    ref = _mlp(xt, ex, 0).numpy()
    _compare(out64, ref, bits)


def test_token_subset_matches_full_evaluation():
    cfg = TINY
    x = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    ex = make_experts_host(cfg)
    sh = make_shared_host(cfg)
    bits, out64 = oracle.moe_forward(x, ids, w, ex, sh)
    sel = np.array([31, 0, 7, 7], np.int64)
    bits_s, out64_s = oracle.moe_forward(x, ids, w, ex, sh, tokens=sel, threads=2)
    assert np.array_equal(bits_s, bits[sel]) and np.array_equal(out64_s, out64[sel])


# --------------------------------------------------------------------------- closed form
def _perm_matrix(perm, n):
    """codes of a 0/1 matrix M[j][perm[j]] = 1.0 (e4m3 code 0x38) -- row j selects input perm[j]."""
    m = np.zeros((n, n), np.uint8)
    m[np.arange(n), perm] = 0x38
    return m


def test_closed_form_permutation_expert():
    """Hand-derivable case, d = d_ff = 128, two experts, K = 2.

    x has three nonzeros x0 = 1.75, x5 = -1, x9 = 0.5, so its group scale is
    1.75/448 = 2^-8 and all three quantise exactly. With gate rows selecting
    pi(j) = (5j + 3) mod 128 and up rows selecting rho = pi o tau (tau cycles
    25 -> 78 -> 26 -> 25), g and u are nonzero only at j = 25, 26, 78:
      g = (1.75, -1, 0.5), u = (0.5, 1.75, -1)
      h = silu(g) u = (0.7454.., -0.4706.., -0.3112..)
    Requantising h with s = fl32(h25/448): codes 448, -288 (282.85 rounds to
    288), -192 (187.04 rounds to 192). The down rows select sigma(o) = (3o + 2)
    mod 128, so y is nonzero at o = 93, 8, 68 (sigma = 25, 26, 78). Expert 1 is
    expert 0 with down scale 2, routing weights (0.75, 0.25): out = 1.25 y.
    A transposed matrix, swapped gate/up or a wrong scale moves or changes these.
    """
    n = 128
    x = np.zeros((1, n), np.float32)
    x[0, 0], x[0, 5], x[0, 9] = 1.75, -1.0, 0.5
    x_bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    j = np.arange(n)
    pi = (5 * j + 3) % n
    tau = j.copy()
    tau[25], tau[26], tau[78] = 78, 25, 26
    rho = pi[tau]
    sigma = (3 * j + 2) % n
    one = np.ones((1, 1), np.float32)
    wg, wu, wd = _perm_matrix(pi, n), _perm_matrix(rho, n), _perm_matrix(sigma, n)
    ex = HostExperts(np.stack([wg, wg]), np.stack([one, one]), np.stack([wu, wu]), np.stack([one, one]),
                     np.stack([wd, wd]), np.stack([one, 2 * one]))
    ids = np.array([[0, 1]], np.int32)
    w = np.array([[0.75, 0.25]], np.float32)
    bits, out64 = oracle.moe_forward(x_bits, ids, w, ex)

    def silu(z):
        return z / (1.0 + math.exp(-z))
    h = np.float32([silu(1.75) * 0.5, silu(-1.0) * 1.75, silu(0.5) * -1.0])
    s = np.float32(h[0]) / np.float32(448.0)
    assert round(float(h[1] / s)) == -283 and round(float(h[2] / s)) == -187
    y = {93: 448.0 * float(s), 8: -288.0 * float(s), 68: -192.0 * float(s)}
    expect = np.zeros(n)
    for o, v in y.items():
        expect[o] = 1.25 * v
    assert np.abs(out64[0] - expect).max() <= 1e-12
    assert np.array_equal(bits[0], oracle.bf16_from_f64(expect))
    assert abs(expect[93] - 1.25 * 0.7454589) < 1e-6


# --------------------------------------------------------------------------- combine algebra
def test_combine_invariants():
    cfg = TINY
    x = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    ex = make_experts_host(cfg)
    _, base = oracle.moe_forward(x, ids, w, ex)
    # scaling all routing weights by 2^3 scales the pre-rounding sum exactly
    _, scaled = oracle.moe_forward(x, ids, w * np.float32(8.0), ex)
    assert np.array_equal(scaled, base * 8.0)
    # a zero weight drops that expert: equals evaluating the token with K-1 experts
    w0 = w.copy()
    w0[:, 2] = 0.0
    _, dropped = oracle.moe_forward(x, ids, w0, ex)
    keep = [0, 1, 3]
    _, fewer = oracle.moe_forward(x, np.ascontiguousarray(ids[:, keep]), np.ascontiguousarray(w[:, keep]), ex)
    assert np.abs(dropped - fewer).max() <= 1e-12 * np.abs(fewer).max()
    # permuting each token's (id, weight) pairs changes only the summation order
    perm = [3, 1, 0, 2]
    _, permuted = oracle.moe_forward(x, np.ascontiguousarray(ids[:, perm]), np.ascontiguousarray(w[:, perm]), ex)
    assert np.abs(permuted - base).max() <= 1e-12 * np.abs(base).max()


def test_shared_expert_alone():
    """All routed weights zero: the output is the shared expert's output on every token."""
    cfg = TINY
    x = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    ex = make_experts_host(cfg)
    sh = make_shared_host(cfg)
    bits, out64 = oracle.moe_forward(x, ids, np.zeros_like(w), ex, sh)
    one_bits, one64 = oracle.moe_forward(x, np.zeros((cfg.N, 1), np.int32), np.ones((cfg.N, 1), np.float32), sh)
    assert np.array_equal(out64, one64) and np.array_equal(bits, one_bits)


def test_oracle_rejects_bad_ids():
    cfg = CONFIGS[0]
    x = make_x_bits(cfg)
    ids, w = make_routing(cfg)
    ex = make_experts_host(cfg)
    bad = ids.copy()
    bad[3, 1] = cfg.E
    with pytest.raises(oracle.OracleError):
        oracle.moe_forward(x, bad, w, ex)
    dup = ids.copy()
    dup[4, 1] = dup[4, 0]
    with pytest.raises(oracle.OracleError):
        oracle.moe_forward(x, dup, w, ex)


def test_expert_rows_against_library_mlp():
    """oracle.expert_rows evaluates one expert on one token per row. Pinned against the torch
    library MLP above (F.linear / F.silu on dequantised weights, float8_e4m3fn activation
    quantisation) for (token, expert) pairs in a scrambled order, with repeats, the last token
    and the last expert: y to 1e-9 relative, and the requantised product h (codes and scales)
    equal to the pinned quantiser applied to torch's float32 h. A wrong token index, expert
    offset or row stride fails it."""
    cfg = Config("rows", 24, 384, 256, 6, 2, "normal", "uniform", "uniform", False, seed=23)
    x = make_x_bits(cfg)
    ex = make_experts_host(cfg)
    rng = np.random.default_rng(24)
    tokens = rng.integers(0, cfg.N, 13)
    experts = rng.integers(0, cfg.E, 13)
    tokens = np.concatenate([tokens, [cfg.N - 1, 0, cfg.N - 1, tokens[0]]]).astype(np.int64)
    experts = np.concatenate([experts, [cfg.E - 1, cfg.E - 1, 0, experts[0]]]).astype(np.int32)
    y, hq, hs = oracle.expert_rows(x, ex, tokens, experts)
    xt = _torch_quant(torch.from_numpy(oracle.bf16_to_f32(x).copy()))
    for i, (t, e) in enumerate(zip(tokens, experts)):
        ref = _mlp(xt[t:t + 1], ex, int(e)).numpy()[0]
        assert np.abs(y[i] - ref).max() <= 1e-9 * np.abs(ref).max()
        g = F.linear(xt[t:t + 1], _dequant_w(ex.w_gate[e], ex.s_gate[e]))
        u = F.linear(xt[t:t + 1], _dequant_w(ex.w_up[e], ex.s_up[e]))
        h = (F.silu(g) * u).to(torch.float32).numpy()
        q_ref, s_ref = oracle.quant_rows_f32(h)
        assert np.array_equal(hq[i], q_ref[0]) and np.array_equal(hs[i], s_ref[0])
    # the same pair gives the same row wherever it appears
    assert np.array_equal(y[0], y[16]) and np.array_equal(hq[0], hq[16])

"""GPU: moe_quantize_rows (the activation quantiser, first step of the grouped SwiGLU
call) must match the oracle bit for bit -- codes and scales."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_ids_amd as moe
import oracle
from parity import bf16_dev, say

pytestmark = pytest.mark.gpu


def _rows(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-20, 20, (rows, 1))).astype(np.float32)
    if rows > 2:
        x[1, :128] = 0.0                       # zero group -> scale 1
        x[2, 128 % cols:128 % cols + 128] = -0.0
    if rows > 3:
        x[3, ::7] *= 1e-30                     # values deep in e4m3's subnormal range after scaling
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rows,cols", [(1, 128), (5, 256), (37, 7168), (1000, 2048), (3, 384)])
def test_quantize_rows_bit_exact(rows, cols):
    rng = np.random.default_rng(rows * 131 + cols)
    bits = _rows(rng, rows, cols)
    say(f"quantize rows={rows} cols={cols}")
    q, s = moe.quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows_bf16(bits)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_e4m3_conversion_exhaustive_over_bf16():
    """Every finite bf16 value v with |v| <= 448, placed in a group whose amax is 448
    (scale exactly 1), so the code is the conversion of v itself."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f32(allb)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    v = allb[keep]
    per = 127
    ngroups = (v.size + per - 1) // per
    pad = ngroups * per - v.size
    v = np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(ngroups, per)
    anchor = np.full((ngroups, 1), 0x43E0, np.uint16)    # bf16 448.0
    bits = np.ascontiguousarray(np.concatenate([anchor, v], axis=1))
    say(f"e4m3 exhaustive groups={ngroups}")
    q, s = moe.quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows_bf16(bits)
    assert np.all(s_ref == 1.0)
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x3FFF, 0x43E0, 0x4000, 0x7F7F, 0x0080, 0x3DCD, 0x1C01, 0x6A5A, 0x0D80],
                         ids=lambda b: f"amax{b:04x}")
def test_quantize_every_bf16_value_against_one_scale(amax_bits):
    """Every finite bf16 value of magnitude at most amax, in groups whose largest magnitude is
    amax: the codes (the quotient v / s rounded by the kernel's corrected reciprocal product, or
    by a plain division for tiny scales) must equal the oracle's, which divides. The amax values
    include scales whose reciprocals are inexact, the largest and smallest normal bf16 and
    scales below 2^-100."""
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f32 = (allb.astype(np.uint32) << 16).view(np.float32)
    amax = np.array([amax_bits << 16], np.uint32).view(np.float32)[0]
    keep = np.isfinite(f32) & (np.abs(f32) <= amax)
    v = allb[keep]
    per = 127
    groups = (v.size + per - 1) // per
    pad = groups * per - v.size
    v = np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(groups, per)
    col = np.full((groups, 1), amax_bits, np.uint16)
    bits = np.concatenate([col, v], axis=1)                    # [groups, 128], first value = amax
    if groups % 8:                                             # 8 groups per row of 1024
        bits = np.concatenate([bits, np.tile(bits[:1], (8 - groups % 8, 1))])
    bits = np.ascontiguousarray(bits.reshape(-1, 1024))
    say(f"quantize every bf16 value, amax bits {amax_bits:#06x}, {bits.shape[0]} rows")
    q, s = moe.quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows_bf16(bits)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _is_nan_code(c: np.ndarray) -> np.ndarray:
    return (np.asarray(c, np.uint8) & 0x7F) == 0x7F


def test_group_with_an_infinity_keeps_finite_codes():
    """A group whose largest magnitude is infinite gets an infinite scale and every finite value
    the code of a signed zero, as the oracle's division gives. The infinite element itself is
    inf / inf, a NaN: both sides give it a NaN code (the format has no infinity; the sign of a
    NaN code carries no value, so only NaN-ness is compared there). The other group of the row
    is unaffected."""
    x = np.linspace(-3, 3, 256, dtype=np.float32).reshape(1, 256)
    x[0, 5] = np.inf
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    say("quantize a group holding an infinity")
    q, s = moe.quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows_bf16(bits)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    finite = np.isfinite(x)
    got = q.cpu().numpy()
    assert np.array_equal(got[finite], q_ref[finite])
    assert _is_nan_code(q_ref[~finite]).all() and _is_nan_code(got[~finite]).all()


def test_nan_inputs_give_nan_codes():
    """NaNs of either sign, among finite values, in groups of several magnitudes: the group scale
    comes from the finite values alone on both sides (a NaN is never the largest magnitude), the
    finite values' codes match bit for bit, and every NaN is encoded as a NaN code, never as a
    saturated +-448 or any other finite code."""
    rng = np.random.default_rng(81)
    x = (rng.standard_normal((6, 512)) * np.exp2(rng.integers(-10, 10, (6, 1)))).astype(np.float32)
    x[0, 3] = np.nan
    x[1, 130] = -np.nan
    x[2, ::5] = np.nan                       # many NaNs in every group of the row
    x[3, :128] = np.nan                      # a group of NaNs only: scale 1, all codes NaN
    x[4, 300] = np.inf                       # an infinity beside a NaN in one group
    x[4, 301] = np.nan
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits[1, 130] |= 0x8000                   # a NaN with the sign bit set
    say("quantize rows holding NaNs")
    q, s = moe.quantize_rows(bf16_dev(bits))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_rows_bf16(bits)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    got = q.cpu().numpy()
    vals = oracle.bf16_to_f32(bits)
    scale = np.repeat(s_ref, 128, axis=1)
    nonfinite = ~np.isfinite(vals) | ~np.isfinite(scale)
    assert np.array_equal(got[~nonfinite], q_ref[~nonfinite])
    nan_in = np.isnan(vals) | (np.isinf(vals) & np.isinf(scale))
    assert _is_nan_code(q_ref[nan_in]).all()
    assert _is_nan_code(got[nan_in]).all(), "a NaN was encoded as a finite code"
    assert np.array_equal(got[nonfinite & ~nan_in], q_ref[nonfinite & ~nan_in])

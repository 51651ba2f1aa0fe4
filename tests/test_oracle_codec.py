"""Pins of the oracle's number formats and quantiser against independent definitions.

The oracle's e4m3 and bfloat16 codecs are written from the format definitions;
here they are checked against torch's float8_e4m3fn / bfloat16 casts (library
codecs that share nothing with the oracle) and against hand-derived values.
The quantiser follows the "Input features" page (evidence "linear":
dynamic activation scheme, fmt e4m3, 128-wide blocks).
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(v, dtype=np.float32))
    return t.clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], ref[~nan])
    # format facts: largest finite 448, smallest subnormal 2^-9, smallest normal 2^-6
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert ours[0x38] == 1.0 and ours[0xB8] == -1.0


def test_encode_all_bf16_patterns_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f32(bits)
    finite = np.isfinite(vals)
    v = vals[finite]
    ours = oracle.e4m3_encode(v)
    ref = _torch_e4m3(v)
    assert np.array_equal(ours, ref)


def test_encode_ties_and_random_floats_match_torch():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = oracle.e4m3_decode(codes)
    hi = oracle.e4m3_decode(codes + 1)
    mids = ((lo + hi) / 2).astype(np.float32)         # exact midpoints (few significant bits)
    assert np.array_equal(mids.astype(np.float64), (lo + hi) / 2)
    rng = np.random.default_rng(1234)
    rnd = (rng.standard_normal(50000) * np.exp2(rng.integers(-14, 10, 50000))).astype(np.float32)
    v = np.concatenate([mids, -mids, rnd, np.float32([448.0, 460.0, 464.0, 1e30, -1e30, 0.0, -0.0])])
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_encode_hand_values():
    # 464 is the midpoint between 448 and the (absent) next step 480: saturates to 448.
    # 2^-10 is the midpoint between 0 and 2^-9: ties to the even code 0.
    # 1.5 * 2^-9 lies between 2^-9 (code 1) and 2^-8 (code 2): ties to code 2.
    # 0.3 = 1.2 * 2^-2 -> mantissa 1.2 * 8 = 9.6 -> nearest 1.25 * 2^-2 (exp field 5, mantissa 2)
    v = np.float32([464.0, 2.0 ** -10, 1.5 * 2.0 ** -9, 0.3, -0.0, 1.0])
    assert list(oracle.e4m3_encode(v)) == [0x7E, 0x00, 0x02, (5 << 3) | 2, 0x80, 0x38]


def test_bf16_from_double_single_rounding():
    # exact tie 1 + 2^-8 between 1 and 1 + 2^-7 -> even (1.0, 0x3F80)
    # just above the tie -> 0x3F81; rounding first to float32 would lose the 2^-40 and give 0x3F80
    assert oracle.bf16_from_f64(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    assert oracle.bf16_from_f64(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert oracle.bf16_from_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82   # tie -> even mantissa 2
    assert oracle.bf16_from_f64(np.array([-2.0]))[0] == 0xC000
    # values exactly representable in float32: one rounding equals torch's float -> bf16 cast
    rng = np.random.default_rng(7)
    f = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f64(f.astype(np.float64)), ref)


def test_quantiser_matches_library_quantiser():
    """Per 128-group: s = fl32(amax/448), q = e4m3(fl32(x/s)); recomputed with torch ops."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((37, 512)) * np.exp2(rng.integers(-6, 6, (37, 1)))).astype(np.float32)
    x[5, 128:256] = 0.0                                 # an all-zero group
    x[6, :128] = -0.0
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.quant_rows_bf16(bits)
    xf = xb.to(torch.float32).reshape(37, 4, 128)
    amax = xf.abs().amax(-1)
    s_ref = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q_ref = (xf / s_ref[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(37, 512)
    assert np.array_equal(s, s_ref.numpy())
    assert np.array_equal(q, q_ref.numpy())


def test_quantiser_properties():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    q, s = oracle.quant_rows_f32(x)
    dec = oracle.e4m3_decode(q).reshape(64, 8, 128)
    # |code| <= 448 and each group's largest magnitude maps to +-448
    assert np.all(np.abs(dec) <= 448.0)
    xg = x.reshape(64, 8, 128)
    arg = np.abs(xg).argmax(-1)
    top = np.take_along_axis(dec, arg[..., None], -1)[..., 0]
    assert np.all(np.abs(top) == 448.0)
    # dequantised error: relative <= 2^-4 for values in the normal range of the scaled format
    deq = dec * s[..., None]
    scaled = np.abs(xg) / s[..., None]
    normal = scaled >= 2.0 ** -6
    rel = np.abs(deq - xg)[normal] / np.abs(xg)[normal]
    assert rel.max() <= 2.0 ** -4
    # subnormal range: absolute error <= half the subnormal step
    assert np.all(np.abs(deq - xg)[~normal] <= 0.5 * 2.0 ** -9 * np.broadcast_to(s[..., None], xg.shape)[~normal] * (1 + 1e-6))
    # zero group: scale 1, zero codes
    qz, sz = oracle.quant_rows_f32(np.zeros((1, 128), np.float32))
    assert sz[0, 0] == 1.0 and np.all(qz == 0)


def test_quantiser_rejects_bad_width():
    with pytest.raises(oracle.OracleError):
        oracle.quant_rows_f32(np.zeros((2, 100), np.float32))


def test_quantiser_nan_reading_against_library_codec():
    """The pages do not speak of NaN; the reading taken is that a NaN has no magnitude (the group
    scale comes from the other values) and is encoded as the NaN code. Pinned against torch's
    codec: scales and the other values' codes equal the torch-op quantiser's on the same rows with
    the NaNs replaced by zeros, and every NaN gets torch's float8_e4m3fn code of NaN. A group of
    NaNs and zeros only has scale 1."""
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((8, 512)) * np.exp2(rng.integers(-6, 6, (8, 1)))).astype(np.float32)
    x[0, 7] = np.nan
    x[1, ::3] = np.nan
    x[2, :128] = np.nan
    x[3, 128:256] = 0.0
    x[3, 130] = np.nan
    x[4, 300] = -np.nan
    q, s = oracle.quant_rows_f32(x)
    nan = np.isnan(x)
    clean = torch.from_numpy(np.where(nan, np.float32(0.0), x)).reshape(8, 4, 128)
    amax = clean.abs().amax(-1)
    s_ref = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q_ref = (clean / s_ref[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(8, 512).numpy()
    assert np.array_equal(s, s_ref.numpy())
    assert np.array_equal(q[~nan], q_ref[~nan])
    nan_code = torch.tensor([float("nan")]).to(torch.float8_e4m3fn).view(torch.uint8).item()
    assert (q[nan] & 0x7F == nan_code & 0x7F).all()
    assert s[2, 0] == 1.0 and s[3, 1] == 1.0

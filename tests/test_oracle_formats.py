"""Pins for the oracle's number formats: bf16, E8M0, MX-FP4 (E2M1), E4M3, NVFP4
and the MXFP8 activation quantiser.

bf16, E8M0 and E4M3 are checked against torch's own dtype conversions; E2M1 against
the format's bit-field definition (sign, two exponent bits with bias 1, one
mantissa bit, subnormals at exponent 0) and the OCP quantiser's error bound.
"""

import numpy as np
import pytest
import torch

from oracle import (E2M1_VALUES, decode_bf16, decode_e4m3, decode_e8m0, decode_mxfp4, decode_nvfp4,
                    quantize_mxfp8, round_e4m3)
from synth import quantize_mxfp4, quantize_nvfp4


def test_bf16_decode_matches_torch(rng):
    v = torch.tensor(rng.normal(size=1000) * 10.0 ** rng.integers(-30, 30, size=1000), dtype=torch.float32)
    b = v.to(torch.bfloat16)
    bits = b.view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(decode_bf16(bits), b.to(torch.float64).numpy())
    specials = torch.tensor([0.0, -0.0, float("inf"), -float("inf")], dtype=torch.bfloat16)
    got = decode_bf16(specials.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(got, [0.0, -0.0, np.inf, -np.inf])
    assert np.signbit(got[1])


def test_e8m0_decode_matches_torch():
    s = np.arange(255, dtype=np.uint8)
    ref = torch.from_numpy(s).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    np.testing.assert_array_equal(decode_e8m0(s), ref)
    assert np.isnan(decode_e8m0(np.array([255], dtype=np.uint8)))[0]


def _e2m1_from_bits(code):
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    return sign * mag


def test_e2m1_table_matches_bit_fields():
    for code in range(16):
        mag = E2M1_VALUES[code & 7]
        assert (-mag if code & 8 else mag) == _e2m1_from_bits(code)


def test_mxfp4_nibble_order_and_scale():
    # byte 0x21: low nibble 1 (0.5) is element 0, high nibble 2 (1.0) element 1
    codes = np.zeros((1, 16), dtype=np.uint8)
    codes[0, 0] = 0x21
    codes[0, 1] = 0xF8        # element 2 = -0.0, element 3 = -6.0
    for s, mult in ((127, 1.0), (130, 8.0), (120, 2.0 ** -7)):
        vals = decode_mxfp4(codes, np.array([[s]], dtype=np.uint8))
        assert vals.shape == (1, 32)
        np.testing.assert_array_equal(vals[0, :4], np.array([0.5, 1.0, -0.0, -6.0]) * mult)
        assert np.signbit(vals[0, 2])
        assert np.all(vals[0, 4:] == 0.0)


def test_mxfp4_all_codes_block():
    codes = np.array([[c | ((c + 1) << 4) for c in range(0, 16, 2)] * 2], dtype=np.uint8)
    vals = decode_mxfp4(codes, np.array([[127]], dtype=np.uint8))
    expect = [_e2m1_from_bits(c) for c in range(16)] * 2
    np.testing.assert_array_equal(vals[0], expect)


def test_mxfp4_blocks_run_along_last_axis():
    codes = np.full((2, 32), 0x22, dtype=np.uint8)   # every element 1.0
    scales = np.array([[127, 128], [126, 131]], dtype=np.uint8)
    vals = decode_mxfp4(codes, scales)
    np.testing.assert_array_equal(vals[0, :32], 1.0)
    np.testing.assert_array_equal(vals[0, 32:], 2.0)
    np.testing.assert_array_equal(vals[1, :32], 0.5)
    np.testing.assert_array_equal(vals[1, 32:], 16.0)


def test_mxfp4_roundtrip_error_bound(rng):
    w = torch.tensor(rng.normal(size=(8, 256)) * 0.02, dtype=torch.float32)
    codes, scales = quantize_mxfp4(w)
    deq = decode_mxfp4(codes.numpy(), scales.numpy())
    wb = w.numpy().astype(np.float64).reshape(8, 8, 32)
    db = deq.reshape(8, 8, 32)
    sc = decode_e8m0(scales.numpy())
    amax = np.abs(wb).max(-1)
    # scale is the largest power of two with amax/scale < 8, i.e. [4, 8)
    assert np.all(amax / sc >= 4) and np.all(amax / sc < 8)
    # in-range elements are within half an E2M1 step (step <= 2 below 6)
    err = np.abs(db - wb) / sc[..., None]
    inrange = np.abs(wb) / sc[..., None] <= 6.0
    steps = np.where(np.abs(wb) / sc[..., None] < 2, 0.5, np.where(np.abs(wb) / sc[..., None] < 4, 1.0, 2.0))
    assert np.all(err[inrange] <= steps[inrange] / 2 + 1e-12)
    # saturated elements decode to +-6 * scale
    sat = ~inrange
    np.testing.assert_array_equal(np.abs(db[sat]), 6.0 * np.broadcast_to(sc[..., None], db.shape)[sat])


def test_mxfp4_values_exact_in_bf16(rng):
    w = torch.tensor(rng.normal(size=(4, 512)) * 0.02, dtype=torch.float32)
    codes, scales = quantize_mxfp4(w)
    deq = decode_mxfp4(codes.numpy(), scales.numpy())
    as_bf16 = torch.tensor(deq).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(deq, as_bf16)


@pytest.mark.parametrize("shape", [(3, 64), (2, 5, 96)])
def test_mxfp4_shapes(shape, rng):
    w = torch.tensor(rng.normal(size=shape), dtype=torch.float32)
    codes, scales = quantize_mxfp4(w)
    assert codes.shape == (*shape[:-1], shape[-1] // 2)
    assert scales.shape == (*shape[:-1], shape[-1] // 32)
    assert decode_mxfp4(codes.numpy(), scales.numpy()).shape == shape


# ----------------------------------------------------------------- NVFP4
# The pages run expert weights in NVFP4 (SGLang-TorchTPU on TPU v7 page,
# "Results"): E2M1 values, one OCP FP8 E4M3 scale per 16 elements, one fp32
# scale per matrix.

def test_e4m3_decode_matches_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = decode_e4m3(b)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9       # largest, smallest subnormal
    assert got[0x38] == 1.0 and got[0xB8] == -1.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_nvfp4_blocks_of_16_and_tensor_scale():
    codes = np.full((2, 16), 0x22, dtype=np.uint8)    # every element 1.0
    scales = np.array([[0x38, 0x40], [0x3C, 0x01]], dtype=np.uint8)  # 1.0, 2.0 | 1.5, 2^-9
    vals = decode_nvfp4(codes, scales, 0.25)
    np.testing.assert_array_equal(vals[0, :16], 0.25)
    np.testing.assert_array_equal(vals[0, 16:], 0.5)
    np.testing.assert_array_equal(vals[1, :16], 0.375)
    np.testing.assert_array_equal(vals[1, 16:], 0.25 * 2.0 ** -9)


def test_nvfp4_reduces_to_e2m1_table():
    codes = np.array([[c | ((c + 1) << 4) for c in range(0, 16, 2)]], dtype=np.uint8)
    vals = decode_nvfp4(codes, np.array([[0x38]], dtype=np.uint8), 1.0)
    np.testing.assert_array_equal(vals[0], [_e2m1_from_bits(c) for c in range(16)])


def test_nvfp4_roundtrip_error_bound(rng):
    w = torch.tensor(rng.normal(size=(8, 256)) * 0.02, dtype=torch.float32)
    codes, scales, ts = quantize_nvfp4(w)
    deq = decode_nvfp4(codes.numpy(), scales.numpy(), ts)
    wb = w.numpy().astype(np.float64)
    # the tensor scale puts the largest block scale at 448
    assert np.isclose(np.abs(wb).max() / (6 * 448), ts, rtol=1e-6)
    sc = decode_e4m3(scales.numpy()) * float(np.float32(ts))
    err = np.abs(deq - wb).reshape(8, 16, 16) / sc[..., None]
    # E2M1 steps are at most 2, and the E4M3 block scale is rounded by at
    # most 1/16 relative, so every element lies within one unit of the block
    assert np.all(err <= 1.0 + 1e-9)
    assert np.linalg.norm(deq - wb) / np.linalg.norm(wb) < 0.12


def test_nvfp4_products_exact_in_bf16(rng):
    """E2M1 x E4M3 has at most 6 significant bits, so a weight without its
    fp32 matrix scale is exact in bf16 (what the MFMA path feeds)."""
    w = torch.tensor(rng.normal(size=(4, 512)) * 0.02, dtype=torch.float32)
    codes, scales, _ = quantize_nvfp4(w)
    deq = decode_nvfp4(codes.numpy(), scales.numpy(), 1.0)
    as_bf16 = torch.tensor(deq).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(deq, as_bf16)


# ----------------------------------------------------------------- MXFP8
# FP8 activations (the pages' "FP8 compute"): E4M3 elements, one E8M0 scale
# per 32 elements along the reduction dimension.

def test_round_e4m3_matches_torch_cast(rng):
    v = rng.normal(size=20000) * 10.0 ** rng.integers(-5, 3, size=20000)
    v = np.concatenate([v, [2.375, -2.375, 2.0 ** -10, 1.5 * 2.0 ** -10, 448.0, 460.0, 464.0, -470.0, 0.0]])
    ref = torch.tensor(v).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_e4m3(v), ref)


def test_mxfp8_block_scale_and_grid(rng):
    v = rng.normal(size=(6, 128)) * 0.3
    q = quantize_mxfp8(v)
    b = v.reshape(6, 4, 32)
    qb = q.reshape(6, 4, 32)
    amax = np.abs(b).max(-1)
    s = np.floor(np.log2(amax)) - 8
    scaled = qb / np.ldexp(1.0, s.astype(int))[..., None]
    # every value is an E4M3 value times the block's power of two
    e4m3 = decode_e4m3(np.arange(256, dtype=np.uint8))
    assert np.isin(scaled, e4m3[~np.isnan(e4m3)]).all()
    # amax / 2**s lies in [256, 512): at most one rounding step plus saturation
    assert np.all(amax / np.ldexp(1.0, s.astype(int)) >= 256)
    err = np.abs(q - v)
    big = np.abs(b).reshape(v.shape) >= np.repeat(np.ldexp(1.0, (s - 6).astype(int)), 32, -1) * 1.0
    assert np.all(err[big] <= np.abs(v)[big] * 2.0 ** -4 + 1e-300)   # half an E4M3 step, normal range


def test_mxfp8_fixed_points_and_zero_block():
    v = np.zeros((1, 64))
    v[0, :32] = [2.0 ** (i % 9) * (1 + (i % 8) / 8) for i in range(32)]   # on the grid
    np.testing.assert_array_equal(quantize_mxfp8(v), v)
    assert np.all(quantize_mxfp8(v)[0, 32:] == 0.0)


def test_swiglu_with_act_quant_reduces_on_grid_inputs(rng):
    from oracle import swiglu_expert
    xs = quantize_mxfp8(rng.normal(size=(3, 64)))
    wg, wu, wd = (rng.normal(size=s) for s in ((32, 64), (32, 64), (64, 32)))
    g = xs @ wg.T
    h = (g / (1 + np.exp(-g))) * (xs @ wu.T)
    np.testing.assert_allclose(swiglu_expert(xs, wg, wu, wd, quantize_mxfp8),
                               quantize_mxfp8(h) @ wd.T, rtol=0, atol=0)


def test_mxfp8_nan_element_stays_nan_and_leaves_the_scale(rng):
    """A NaN element quantises to NaN, and the block's other elements are
    quantised exactly as if it were absent: a block with a NaN in place of a
    value no larger than its amax gives the same values elsewhere as the block
    with that position set to zero (which cannot change amax)."""
    v = rng.normal(size=(4, 64)) * 3.0
    with_nan = v.copy()
    with_nan[1, 5] = np.nan
    with_nan[3, 40] = np.nan
    zeroed = v.copy()
    zeroed[1, 5] = 0.0
    zeroed[3, 40] = 0.0
    for r, c in ((1, 5), (3, 40)):   # the replaced value is not the block maximum
        blk = v[r, (c // 32) * 32:(c // 32 + 1) * 32]
        assert abs(v[r, c]) < np.abs(blk).max()
    qn = quantize_mxfp8(with_nan)
    qz = quantize_mxfp8(zeroed)
    assert np.isnan(qn[1, 5]) and np.isnan(qn[3, 40])
    assert np.isnan(qn).sum() == 2
    keep = ~np.isnan(qn)
    np.testing.assert_array_equal(qn[keep], qz[keep])
    # an all-NaN block: every element NaN, the rest of the row untouched
    allnan = v.copy()
    allnan[0, :32] = np.nan
    q = quantize_mxfp8(allnan)
    assert np.isnan(q[0, :32]).all()
    np.testing.assert_array_equal(q[0, 32:], quantize_mxfp8(v)[0, 32:])

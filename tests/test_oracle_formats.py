"""Pins of the oracle's number formats against torch's casts and the format definitions."""
import numpy as np
import pytest
import torch

from oracle import formats


def _torch_bf16(v32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(v32).to(torch.bfloat16).float().double().numpy()


def test_bf16_matches_torch_cast_on_binary32_inputs():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),  # subnormals
        (rng.standard_normal(20000) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.3895314e38], np.float32),
    ])
    got = formats.round_to_bf16(v.astype(np.float64))
    exp = _torch_bf16(v)
    np.testing.assert_array_equal(got, exp)


def test_bf16_rounds_float64_once_not_through_binary32():
    # 1 + 2^-8 is the exact midpoint between 1 and 1 + 2^-7: ties to even (1.0).
    assert formats.round_to_bf16(1.0 + 2.0 ** -8) == 1.0
    # Just above the midpoint must round up; going through binary32 first would
    # lose the 2^-40 and tie down to 1.0 (double rounding).
    assert formats.round_to_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert formats.round_to_bf16(-(1.0 + 3 * 2.0 ** -8)) == -(1.0 + 2 * 2.0 ** -7)


def test_bf16_bits_decode_and_encode_roundtrip():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = formats.bf16_bits_to_f64(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(t))
    fin = np.isfinite(vals)
    np.testing.assert_array_equal(vals[fin], t[fin])
    # every finite bf16 value encodes back to its own bits (except -0/+0 keep sign)
    enc = formats.f64_to_bf16_bits(vals[fin])
    np.testing.assert_array_equal(enc, bits[fin])


def test_e4m3_table_matches_torch_float8_decode():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    t = codes.view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(np.isnan(formats.E4M3_VALUES), np.isnan(t))
    fin = ~np.isnan(t)
    np.testing.assert_array_equal(formats.E4M3_VALUES[fin], t[fin])
    assert np.nanmax(formats.E4M3_VALUES) == 448.0
    assert formats.E4M3_VALUES[1] == 2.0 ** -9  # smallest subnormal


def test_e4m3_encode_matches_torch_float8_cast():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.uniform(-448, 448, 100000),
        rng.standard_normal(100000) * 0.01,  # subnormal range
        rng.standard_normal(100000) * 30,
        # exact midpoints between neighbouring codes (ties to even)
        (formats.E4M3_VALUES[1:126] + formats.E4M3_VALUES[2:127]) / 2,
        np.array([0.0, 448.0, 450.0, 464.0, -464.0]),
    ]).astype(np.float32)
    got = formats.e4m3_encode(v.astype(np.float64))
    exp = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, exp)
    assert formats.e4m3_encode(np.array([470.0]))[0] & 0x7F == 0x7F  # beyond 464 -> NaN


def test_every_e4m3_value_is_a_bf16_value():
    fin = formats.E4M3_VALUES[~np.isnan(formats.E4M3_VALUES)]
    np.testing.assert_array_equal(formats.round_to_bf16(fin), fin)


@pytest.mark.parametrize("seed", [0, 1])
def test_e4m3_row_quantiser_invariants(seed):
    rng = np.random.default_rng(seed)
    r = (rng.standard_normal((500, 64)) * rng.uniform(0.01, 10, (500, 1))).astype(np.float32)
    r[7] = 0.0
    codes, scale, stored = formats.e4m3_quantize_rows(r)
    assert scale.dtype == np.float32 and scale[7] == 1.0 and np.all(codes[7] & 0x7F == 0)
    vals = formats.e4m3_decode(codes)
    nz = np.arange(500) != 7
    # the absmax element of each non-zero row lands on +-448
    np.testing.assert_array_equal(np.max(np.abs(vals[nz]), axis=1), 448.0)
    # reconstruction error at most half a code step (relative 2^-4), plus subnormal floor
    err = np.abs(stored - r.astype(np.float64))
    bound = np.maximum(np.abs(r) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # scale is the binary32 quotient of the row absmax by 448
    np.testing.assert_array_equal(scale[nz], np.max(np.abs(r[nz]), axis=1) / np.float32(448.0))


def test_e4m3_row_quantiser_tiny_and_nonfinite_rows():
    """Rows whose absmax quotient underflows take scale 1 (like an all-zero row)
    instead of dividing by 0; a NaN element is left out of the absmax and gets
    the NaN code; an infinite element makes its whole stored row NaN."""
    sub = np.float32(2.0 ** -149)
    r = np.array([
        [sub, -3 * sub, 0.0, 0.0],           # absmax 3 * 2^-149: 3 * 2^-149 / 448 underflows to 0
        [2.0 ** -120, 1.0, -2.0, 0.5],       # ordinary row
        [np.nan, 1.0, -448.0 * 2, 0.25],     # NaN element
        [np.inf, 1.0, 0.0, -1.0],            # infinite element
    ], dtype=np.float32)
    codes, scale, stored = formats.e4m3_quantize_rows(r)
    assert scale[0] == 1.0 and np.all(codes[0] & 0x7F == 0) and np.all(np.isfinite(stored[0]))
    assert scale[1] == np.float32(2.0) / np.float32(448.0)
    assert scale[2] == np.float32(896.0) / np.float32(448.0) == 2.0
    assert codes[2, 0] & 0x7F == 0x7F and np.isnan(stored[2, 0]) and np.all(np.isfinite(stored[2, 1:]))
    np.testing.assert_array_equal(stored[2, 1:], [1.0, -896.0, 0.25])
    assert np.isposinf(scale[3]) and np.all(np.isnan(stored[3]))
    # torch's own e4m3 conversion agrees on the codes of the finite rows
    y = (r[:3] / scale[:3, None]).astype(np.float32)
    fin = ~np.isnan(y)
    exp = torch.from_numpy(np.where(fin, y, 0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(codes[:3][fin], exp[fin])

"""Pins for the oracle's stored-format codecs (fp32 / bf16 / OCP E4M3).

Independent references: torch's own float8_e4m3fn and bfloat16 conversions
(library routines), and constants fixed by the OCP 8-bit floating point
specification (bias 7, largest finite 448, smallest normal 2**-6, smallest
subnormal 2**-9, NaN pattern S.1111.111).
"""
import numpy as np
import pytest
import torch

from oracle import codec


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = codec.e4m3_value_table()
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e4m3_spec_constants():
    v = codec.e4m3_value_table()
    assert v[0x7E] == 448.0                 # largest finite
    assert v[0x08] == 2.0 ** -6             # smallest normal
    assert v[0x01] == 2.0 ** -9             # smallest subnormal
    assert v[0x38] == 1.0                   # exponent field 7 = bias
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert np.all(np.diff(v[:127]) > 0)     # positive codes ascend


def test_e4m3_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(50000) * 40, rng.standard_normal(50000) * 1e-2,
        rng.uniform(-463.9, 463.9, 20000),
        # exact midpoints between neighbouring codes: ties must go to even
        ((codec.e4m3_value_table()[1:126] + codec.e4m3_value_table()[2:127]) / 2),
    ]).astype(np.float32)
    ours = codec.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    x = np.float32([448.0, 449.0, 470.0, 1e9, -1e9, -0.0, -1e-30, 0.0])
    c = codec.e4m3_encode(x)
    assert c.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00]


def test_e4m3_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(codec.e4m3_encode(codec.e4m3_decode(codes)), codes)


def test_bf16_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(100000) * 3, rng.standard_normal(1000) * 1e-30]).astype(np.float32)
    # exact bf16 midpoints
    mid = (np.arange(0x3F800000, 0x3F800000 + 2000 * 0x10000, 0x10000, dtype=np.uint32) + 0x8000)
    x = np.concatenate([x, mid.view(np.float32)])
    ours = codec.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = codec.bf16_decode(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_quantize_rep_error_bound(dtype):
    rng = np.random.default_rng(2)
    for _ in range(50):
        c = (rng.standard_normal(128) * rng.uniform(0.01, 10)).astype(np.float32)
        raw, sc = codec.quantize_rep(c, dtype)
        v = codec.decode_codes(raw, dtype).astype(np.float64) * float(sc)
        amax = float(np.max(np.abs(c)))
        if dtype == "f32":
            assert np.array_equal(v, c.astype(np.float64))
        elif dtype == "bf16":
            assert np.all(np.abs(v - c) <= np.abs(c) * 2.0 ** -8)   # unit roundoff of an 8-bit significand
        else:
            assert sc == np.float32(np.float32(amax) / np.float32(448.0))
            # the largest element maps to (about) 448, normals carry 3 mantissa bits
            assert np.max(np.abs(codec.e4m3_decode(raw))) >= 416.0
            assert np.all(np.abs(v - c) <= np.maximum(np.abs(c) * 2.0 ** -4, float(sc) * 2.0 ** -10) * 1.0001)


def test_quantize_rep_zero_centroid():
    raw, sc = codec.quantize_rep(np.zeros(32, np.float32), "e4m3")
    assert sc == 1.0 and not raw.any()

"""Pins of the oracle's E4M3 codec and 1x128 scaling rule: the format's
definition, torch's float8_e4m3fn conversion (a library routine) on all
codes and on random values, round-to-nearest-even at every midpoint, and
saturation."""
import numpy as np
import torch

import oracle
from oracle import e4m3_decode, e4m3_encode


def test_decode_known_codes():
    assert e4m3_decode(np.array([0x38]))[0] == 1.0
    assert e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert e4m3_decode(np.array([0xFE]))[0] == -448.0
    assert e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6      # smallest normal
    assert e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9      # smallest subnormal
    assert e4m3_decode(np.array([0x07]))[0] == 7 * 2.0 ** -9  # largest subnormal
    assert np.isnan(e4m3_decode(np.array([0x7F, 0xFF]))).all()
    assert np.signbit(e4m3_decode(np.array([0x80]))[0])


def test_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().double().numpy()
    got = e4m3_decode(codes)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    np.testing.assert_array_equal(got[~both_nan], ref[~both_nan])
    np.testing.assert_array_equal(np.signbit(got[~both_nan]), np.signbit(ref[~both_nan]))


def test_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert np.array_equal(e4m3_encode(e4m3_decode(codes)), codes)


def test_midpoints_round_to_even():
    vals = e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (vals[:-1] + vals[1:]) / 2                  # exact in fp64
    got = e4m3_encode(mids)
    lower = np.arange(0, 0x7E)
    expect = np.where(lower % 2 == 0, lower, lower + 1)
    np.testing.assert_array_equal(got, expect)
    # just off the midpoint rounds to the nearer neighbour
    np.testing.assert_array_equal(e4m3_encode(np.nextafter(mids, 0)), lower)
    np.testing.assert_array_equal(e4m3_encode(np.nextafter(mids, 1e9)), lower + 1)
    # 272 lies halfway between 256 (mantissa 000) and 288 (001): goes to 256
    assert e4m3_encode(np.array([272.0]))[0] == 0x78


def test_saturation_and_signs():
    np.testing.assert_array_equal(e4m3_encode(np.array([448.0, 449.0, 464.0, 1e9, np.inf])), [0x7E] * 5)
    np.testing.assert_array_equal(e4m3_encode(np.array([-448.0, -500.0, -np.inf])), [0xFE] * 3)
    np.testing.assert_array_equal(e4m3_encode(np.array([-1e-12, 0.0, -0.0, 1e-12])), [0x80, 0x00, 0x80, 0x00])
    assert e4m3_encode(np.array([np.nan]))[0] == 0x7F


def test_encode_matches_torch_on_random_fp32():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.normal(size=200000) * 50,
        rng.uniform(-2 ** -5, 2 ** -5, size=100000),       # subnormal range
        rng.uniform(-463.9, 463.9, size=100000),
    ]).astype(np.float32)
    v = v[np.abs(v) < 464]                                # torch turns |v| >= 464 into NaN
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(e4m3_encode(v.astype(np.float64)), ref)


def test_quantize_1x128_rule():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(5, 384)).astype(np.float32)
    v[1, 128:256] = 0.0
    v[3, :128] *= 1e-6
    codes, scales = oracle.quantize_1x128(v)
    assert codes.shape == (5, 384) and scales.shape == (5, 3) and scales.dtype == np.float32
    assert scales[1, 1] == 1.0 and not codes[1, 128:256].any()
    for r in range(5):
        for t in range(3):
            tile = v[r, t * 128:(t + 1) * 128]
            amax = np.abs(tile).max()
            if amax == 0:
                continue
            assert scales[r, t] == np.float32(amax / np.float32(448.0))
            i = np.abs(tile).argmax()
            assert codes[r, t * 128 + i] & 0x7F == 0x7E      # the largest element maps to +-448
    deq = oracle.dequantize_1x128(codes, scales)
    # error bound: half an E4M3 ulp, relative 2^-4 in the normal range, absolute
    # 2^-10 * scale in the subnormal range
    err = np.abs(deq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * np.repeat(scales, 128, axis=1)) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_dequantize_blocks():
    codes = np.full((256, 128), 0x38, np.uint8)         # every code is 1.0
    scales = np.array([[2.0], [0.5]], np.float32)
    w = oracle.dequantize_blocks(codes, scales)
    assert np.all(w[:128] == 2.0) and np.all(w[128:] == 0.5)

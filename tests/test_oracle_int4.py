"""Pins of the oracle's 4-bit weight decoder: the two's-complement field
definition checked against sign extension by arithmetic shift (an independent
route) on every byte, a hand-worked packing example, the group-to-scale
mapping, and the input generator's rounding rule."""
import json
import os

import numpy as np
import torch

import oracle
from moe_inputs import int4_group_quantize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "int4_packing_example.json")


def test_decode_matches_arithmetic_shift_on_every_byte():
    b = np.arange(256, dtype=np.uint8)
    got = oracle.unpack_int4(b.reshape(1, 256))[0]
    lo = (b << 4).astype(np.uint8).view(np.int8).astype(np.int64) >> 4    # sign-extend bits 0-3
    hi = b.view(np.int8).astype(np.int64) >> 4                             # sign-extend bits 4-7
    np.testing.assert_array_equal(got[0::2], lo)
    np.testing.assert_array_equal(got[1::2], hi)
    assert got.min() == -8 and got.max() == 7


def test_decode_field_values():
    assert oracle.int4_decode(np.arange(16)).tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_packing_example():
    with open(GOLDEN) as f:
        fx = json.load(f)
    packed = np.array(fx["bytes"], dtype=np.uint8).reshape(1, -1)
    assert oracle.unpack_int4(packed)[0].tolist() == fx["values"]


def test_group_scale_mapping():
    # q = 1 everywhere (byte 0x11): the dequantised weight is the scale of its
    # (row, 128-column group), broadcast over the group.
    rows, cols = 3, 384
    packed = np.full((rows, cols // 2), 0x11, np.uint8)
    s = np.array([[1.0, 2.0, 4.0], [0.5, -3.0, 8.0], [7.0, 0.25, 1.5]], np.float32)   # (group, row)
    w = oracle.dequantize_int4_groups(packed, s)
    for r in range(rows):
        for c in (0, 1, 126, 127, 128, 129, 255, 256, 383):
            assert w[r, c] == s[c // 128, r]


def test_dequantize_is_code_times_scale():
    rng = np.random.default_rng(5)
    packed = rng.integers(0, 256, size=(4, 128), dtype=np.uint8)        # 256 columns
    s = rng.standard_normal((2, 4)).astype(np.float32)
    w = oracle.dequantize_int4_groups(packed, s)
    for r in range(4):
        for j in range(128):
            byte = int(packed[r, j])
            for half, c in ((0, 2 * j), (1, 2 * j + 1)):
                n = (byte >> (4 * half)) & 0xF
                q = n - 16 if n >= 8 else n
                assert w[r, c] == q * float(s[c // 128, r])


def test_generator_rounding_rule():
    # The input generator's codes decode to within half a step of the fp32
    # weight, the largest magnitude of a group maps to +-7, codes stay in
    # [-7, 7], and an all-zero group gets scale 1 and codes 0.
    g = torch.Generator().manual_seed(3)
    w = torch.randn(5, 512, generator=g) * 0.02
    w[2, 128:256] = 0.0
    packed, scales = int4_group_quantize(w)
    assert packed.shape == (5, 256) and packed.dtype == torch.uint8
    assert scales.shape == (4, 5) and scales.dtype == torch.float32
    q = oracle.unpack_int4(packed.numpy())
    deq = oracle.dequantize_int4_groups(packed.numpy(), scales.numpy())
    s = np.repeat(scales.numpy().T.astype(np.float64), 128, axis=1)
    assert np.all(np.abs(deq - w.double().numpy()) <= 0.5 * s * (1 + 1e-6))
    assert q.min() >= -7 and q.max() <= 7
    gq = np.abs(q.reshape(5, 4, 128)).max(axis=-1)                 # (row, group)
    assert np.all(gq[scales.numpy().T != 1.0] == 7)
    assert scales[1, 2].item() == 1.0 and np.all(q[2, 128:256] == 0)

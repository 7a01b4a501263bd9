"""Pins of the oracle's FP8 path beyond the E4M3 codec itself:

* the 128x128 weight-block scale layout, on several blocks along both axes
  (FP8 routing post, FP8 section: 128x128 weight blocks; V3 lab page §3
  infer.toml weight_block_size [128, 128]);
* how the layer composes the 1x128 activation rule: x is quantised once and
  that image feeds the routed experts and the shared expert, the router reads
  the unquantised x (walkthrough §8: the gate is not quantised), and the
  intermediate is quantised after SiLU(gate) * up, not gate and up apart.

The layer case is built by hand so that every intermediate value is exact and
the expected output is a handful of integers: a plausible mistake in the
composition changes one of them."""
import numpy as np
import pytest

import oracle
from oracle import e4m3_decode


def test_dequantize_blocks_maps_every_block_to_its_scale():
    rng = np.random.default_rng(7)
    N, K = 384, 256                                   # 3 x 2 blocks: both block axes exercised, not square
    codes = rng.integers(0, 256, size=(N, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38              # no NaN codes
    scales = np.array([[1.0, 3.0], [0.5, 0.25], [7.0, 1.5]], np.float32)
    w = oracle.dequantize_blocks(codes, scales)
    assert w.shape == (N, K)
    vals = e4m3_decode(codes)
    for n in range(0, N, 17):                         # element by element on a grid that crosses every block
        for k in range(0, K, 13):
            assert w[n, k] == vals[n, k] * float(scales[n // 128, k // 128])
    # a whole block at a time: block (bn, bk) is its codes times its own scale
    for bn in range(3):
        for bk in range(2):
            blk = np.s_[bn * 128:(bn + 1) * 128, bk * 128:(bk + 1) * 128]
            np.testing.assert_array_equal(w[blk], vals[blk] * float(scales[bn, bk]))


def test_quantize_dequantize_is_the_tile_rule():
    # one tile: amax 448 fixes the scale at exactly 1, so the image is the E4M3
    # rounding of every value: 1.0625 is the midpoint of 1 and 1.125 (to 1,
    # even mantissa), 29.75 lies between 28 and 30 (to 30)
    v = np.zeros((1, 128))
    v[0, :4] = [448.0, 1.0625, 29.75, -3.0]
    got = oracle.quantize_dequantize_1x128(v)
    np.testing.assert_array_equal(got[0, :4], [448.0, 1.0, 30.0, -3.0])
    assert not got[0, 4:].any()


# ------------------------------------------------------------ hand-built layer ---
#
# H = I = Is = 128, E = 2, k = 1, softmax, norm, scale 1, one token.  Every
# weight is an E4M3 value (block scale 1).  x has amax 448, so its 1x128 scale
# is 1 and Q(x) rounds each entry to E4M3:
#   x[0] = 448 -> 448,  x[1] = 1.0625 -> 1 (tie to even),  x[2] = 1.03125 -> 1,
#   x[3] = 1 -> 1,      x[4] = 2 -> 2.
# Router: logit_0 = x[2], logit_1 = x[1].  On the raw x expert 1 wins
# (1.0625 > 1.03125); on Q(x) both logits are 1 and the tie would go to expert 0.
# Expert 1 (SiLU(v) equals v in fp32 for v >= 28):
#   g0 = 28 x3, u0 = 16 x3              -> h0 = 448: the intermediate's scale is 1
#   g1 = 32 x3 + x4 = 34, u1 = x3 / 32   -> h1 = 1.0625 -> Q(h1) = 1
#   g2 = 28 x3, u2 = x1                 -> h2 = 28 on Q(x) (29.75 -> 30 on raw x)
#   y[10] = Q(h1), y[11] = Q(h2), y[12] = Q(h0)
# Expert 0 writes only y[13] = 448.  Shared expert:
#   g0 = 28 x3, u0 = 16 x3 -> 448;  g1 = 28 x3, u1 = x1 -> 28 on Q(x) (30 on raw x)
#   sh[20] = Q(h1), sh[21] = Q(h0)
# So out = 1 at column 10, 28 at 11, 448 at 12, 28 at 20, 448 at 21, 0 elsewhere.
# Quantising gate and up apart instead of h moves column 12 (gate's tile scale
# is then 34/448, and 28 is not a multiple of it); skipping the intermediate's
# quantisation leaves 1.0625 in column 10.

H = I = IS = 128


def _hand_layer():
    x = np.zeros((1, H))
    x[0, :5] = [448.0, 1.0625, 1.03125, 1.0, 2.0]
    gate_w = np.zeros((2, H))
    gate_w[0, 2] = 1.0
    gate_w[1, 1] = 1.0
    w13 = np.zeros((2, 2 * I, H))
    w2 = np.zeros((2, H, I))
    # expert 1
    w13[1, 0, 3], w13[1, I + 0, 3] = 28.0, 16.0
    w13[1, 1, 3], w13[1, 1, 4], w13[1, I + 1, 3] = 32.0, 1.0, 1.0 / 32
    w13[1, 2, 3], w13[1, I + 2, 1] = 28.0, 1.0
    w2[1, 10, 1] = w2[1, 11, 2] = w2[1, 12, 0] = 1.0
    # expert 0
    w13[0, 0, 3], w13[0, I + 0, 3] = 28.0, 16.0
    w2[0, 13, 0] = 1.0
    # shared expert
    sh13 = np.zeros((2 * IS, H))
    sh2 = np.zeros((H, IS))
    sh13[0, 3], sh13[IS + 0, 3] = 28.0, 16.0
    sh13[1, 3], sh13[IS + 1, 1] = 28.0, 1.0
    sh2[20, 1] = sh2[21, 0] = 1.0
    return x, gate_w, w13, w2, sh13, sh2


def _expected():
    out = np.zeros((1, H))
    out[0, [10, 11, 12, 20, 21]] = [1.0, 28.0, 448.0, 28.0, 448.0]
    return out


def test_hand_layer_weights_are_e4m3_values():
    # the construction only uses values the weight format holds exactly (block scale 1)
    _, _, w13, w2, sh13, sh2 = _hand_layer()
    for w in (w13, w2, sh13, sh2):
        v = np.unique(w)
        np.testing.assert_array_equal(e4m3_decode(oracle.e4m3_encode(v)), v)


def test_fp8_composition_whole_layer():
    x, gate_w, w13, w2, sh13, sh2 = _hand_layer()
    q = oracle.quantize_dequantize_1x128
    out, info = oracle.moe_layer(x, gate_w, None, w13, w2, sh13, sh2, scoring="softmax", top_k=1,
                                 norm_topk_prob=True, routed_scaling_factor=1.0, quantize_x=q, quantize_h=q)
    assert info["ids"].tolist() == [[1]]               # the router saw the raw x
    assert info["w"].tolist() == [[1.0]]
    np.testing.assert_array_equal(out, _expected())


def test_fp8_composition_selected_rows():
    x, _, w13, w2, sh13, sh2 = _hand_layer()
    q = oracle.quantize_dequantize_1x128
    out = oracle.moe_layer_rows([0], x, np.array([[1]]), np.array([[1.0]]), lambda e: (w13[e], w2[e]),
                                lambda: (sh13, sh2), quantize_x=q, quantize_h=q)
    np.testing.assert_array_equal(out, _expected())


@pytest.mark.parametrize("which", ["x", "h"])
def test_hand_layer_depends_on_each_quantisation(which):
    # the case is sharp: leaving either quantisation out changes the output
    x, gate_w, w13, w2, sh13, sh2 = _hand_layer()
    q = oracle.quantize_dequantize_1x128
    kw = dict(quantize_x=None if which == "x" else q, quantize_h=None if which == "h" else q)
    out, _ = oracle.moe_layer(x, gate_w, None, w13, w2, sh13, sh2, scoring="softmax", top_k=1,
                              norm_topk_prob=True, routed_scaling_factor=1.0, **kw)
    assert not np.array_equal(out, _expected())

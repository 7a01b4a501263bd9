"""FP8 E4M3 encoding and the 1x128 / 128x128 scaling rules (test infrastructure only).

Format: OCP E4M3FN - 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
no infinities, S.1111.111 is NaN, largest finite magnitude 448.  The pages
name E4M3 with 1x128 activation tiles and 128x128 weight blocks, scaled
dynamically (MoA routing + FP8 inference, blog.hotdry.top, FP8 section;
V3 lab page, gsyq.cn/news/313569, §3 infer.toml [fp8]).

Readings taken where the pages are silent:
  * symmetric scaling with no zero point and no clipping: a tile's scale is
    fp32(amax / 448), so the tile's largest magnitude maps to 448 exactly;
  * an all-zero tile gets scale 1 and codes 0;
  * v / scale is one correctly rounded fp32 division; the fp32 quotient is
    rounded to E4M3 to nearest, ties to even mantissa, magnitudes at or above
    448 saturate to 448, the sign is kept (so tiny negatives become -0).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def _decode_from_fields(c: np.ndarray) -> np.ndarray:
    """Value of codes c from the bit fields of the format."""
    c = np.asarray(c).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = c & 0x7
    subnormal = man / 8.0 * 2.0 ** -6
    normal = (1.0 + man / 8.0) * np.exp2(exp - 7.0)
    mag = np.where(exp == 0, subnormal, normal)
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return sign * mag


_TABLE = _decode_from_fields(np.arange(256))                 # all 256 codes, fp64


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Exact fp64 value of every E4M3FN code (NaN for the two NaN codes),
    looked up in the table of all 256 codes built from the bit fields."""
    return _TABLE[np.asarray(codes, np.uint8)]


_POS_CODES = np.arange(0, 0x7F, dtype=np.uint8)          # 0 .. 126: all finite non-negatives
_POS_VALUES = e4m3_decode(_POS_CODES)                      # strictly increasing, 0 .. 448


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Round real values (exact in fp64) to E4M3FN codes: nearest finite value,
    ties to the even code (even mantissa), |v| >= 448 -> 448, NaN -> 0x7F."""
    v = np.asarray(v, np.float64)
    mag = np.abs(v)
    sat = np.minimum(mag, E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, sat, side="left")     # first value >= sat
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - sat
    d_lo = sat - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quantize_1x128(v: np.ndarray):
    """Dynamic 1x128 tile quantisation of a (rows, cols) activation, cols a
    multiple of 128, evaluated in fp32: per (row, tile) amax of |v|, scale =
    fp32(amax / 448) (1 when amax = 0), code = E4M3(fp32(v / scale)).
    Returns (codes uint8 (rows, cols), scales float32 (rows, cols/128))."""
    v32 = np.asarray(v, np.float32)
    R, C = v32.shape
    if C % 128:
        raise ValueError("1x128 quantisation needs a multiple of 128 columns")
    tiles = v32.reshape(R, C // 128, 128)
    amax = np.abs(tiles).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (tiles / scale[..., None]).astype(np.float32)
    return e4m3_encode(q).reshape(R, C), scale


def dequantize_1x128(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code value * tile scale, fp64."""
    R, C = codes.shape
    return (e4m3_decode(codes).reshape(R, C // 128, 128)
            * np.asarray(scales, np.float64)[..., None]).reshape(R, C)


def quantize_dequantize_1x128(v: np.ndarray) -> np.ndarray:
    """The value an FP8 GEMM operand carries: v quantised per 1x128 tile by
    quantize_1x128 (after its fp32 cast) and decoded back, fp64.  This is the
    step applied to x before both expert GEMM inputs and to h after SiLU*up."""
    return dequantize_1x128(*quantize_1x128(np.asarray(v, np.float64)))


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(N,K) weight from E4M3 codes and one fp32 scale per 128x128 block, fp64:
    w[n, k] = value(codes[n, k]) * scales[n // 128, k // 128], scales (N/128, K/128)."""
    N, K = codes.shape
    v = e4m3_decode(codes).reshape(N // 128, 128, K // 128, 128)
    return (v * np.asarray(scales, np.float64)[:, None, :, None]).reshape(N, K)

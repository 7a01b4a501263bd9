"""Signed 4-bit expert weights with one fp32 scale per row and 128 input
columns (test infrastructure only).

The pages name the format only: expert FFN weights stored in 4 bits with
16-bit activations (W4A16), the router left unquantised (MoE inference
walkthrough, zhiyuanblog.org/blog/moe-inference, §8 MoE quantisation table).
Readings taken where they are silent:
  * a weight is a two's-complement 4-bit integer q in [-8, 7] times a scale;
  * a weight matrix stored (out, in) packs two consecutive input columns per
    byte, the even column in the low nibble (bits 0-3), the odd one in the
    high nibble (bits 4-7): packed shape (out, in/2), uint8;
  * one fp32 scale per output row and per group of 128 consecutive input
    columns (the 128-wide granularity the FP8 recipe uses for activation
    tiles), stored group-major as 4-bit checkpoints commonly store them:
    scales shape (in/128, out); value = q * scale, exact in fp64;
  * activations stay in the activation dtype (bf16) and are not quantised.
"""
from __future__ import annotations

import numpy as np

INT4_GROUP = 128


def int4_decode(nibbles: np.ndarray) -> np.ndarray:
    """Value of 4-bit two's-complement fields 0..15: n for n < 8, n - 16 otherwise."""
    n = np.asarray(nibbles).astype(np.int64) & 0xF
    return np.where(n >= 8, n - 16, n)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """(rows, cols/2) packed bytes -> (rows, cols) int64 values; column 2j is
    the low nibble of byte j, column 2j+1 the high nibble."""
    b = np.asarray(packed, np.uint8)
    rows, half = b.shape
    out = np.empty((rows, 2 * half), np.int64)
    out[:, 0::2] = int4_decode(b & 0xF)
    out[:, 1::2] = int4_decode(b >> 4)
    return out


def dequantize_int4_groups(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(rows, cols) fp64 weight: q[r, c] * scales[c // 128, r]."""
    q = unpack_int4(packed)
    rows, cols = q.shape
    if cols % INT4_GROUP:
        raise ValueError("4-bit weights need a multiple of 128 input columns")
    s = np.asarray(scales, np.float64)
    if s.shape != (cols // INT4_GROUP, rows):
        raise ValueError(f"scales shape {s.shape}, need {(cols // INT4_GROUP, rows)}")
    return (q.reshape(rows, cols // INT4_GROUP, INT4_GROUP) * s.T[:, :, None]).reshape(rows, cols)

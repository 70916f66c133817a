"""Scalar definitions of the element formats, plus table-driven numpy versions.

Test infrastructure (see oracle/__init__.py).

Sources:
  * FP8 E4M3 as PyTorch's float8_e4m3fn: the KV pool dtype on "The FP8 KV Cache Wall"
    (section "Context and Motivation") and on "The Smoking Gun" (dtype pair
    BFloat16 / Float8_e4m3fn).  Read as the OCP 8-bit E4M3 format: bias 7, no
    infinities, NaN only at S.1111.111, largest finite value 448.
  * E2M1: "1 sign + 2 exponent + 1 mantissa" (NVFP4 article, format section).  Read as
    the OCP 4-bit E2M1 format: bias 1, subnormal at exponent 0, no inf/NaN, largest 6.
  * The calibrated global scale amax / (6 * 448) of the NVFP4 workloads fixes 6 and 448
    as the largest magnitudes of the two formats.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def e4m3_decode(code: int) -> float:
    """Value of an e4m3fn byte: sign bit 7, exponent bits 6-3 (bias 7), mantissa bits 2-0."""
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        mag = (m / 8.0) * 2.0 ** -6
    else:
        mag = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e2m1_decode(code: int) -> float:
    """Value of an E2M1 nibble: sign bit 3, exponent bits 2-1 (bias 1), mantissa bit 0."""
    s = (code >> 3) & 1
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        mag = 0.5 * m
    else:
        mag = (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return -mag if s else mag


# Non-negative finite grids, indexed by the magnitude code (sign bit clear).
E4M3_GRID = [e4m3_decode(c) for c in range(0x7F)]      # codes 0x00..0x7E
E2M1_GRID = [e2m1_decode(c) for c in range(0x8)]       # codes 0x0..0x7


def _nearest_even(a: float, grid: list[float]) -> int:
    """Index of the grid value nearest to a >= 0; on a tie the even index wins (the even
    index is the one whose mantissa LSB is 0).  Values above the largest grid point
    saturate to it."""
    if a >= grid[-1]:
        return len(grid) - 1
    best = 0
    best_d = abs(a - grid[0])
    for k in range(1, len(grid)):
        d = abs(a - grid[k])
        if d < best_d or (d == best_d and k % 2 == 0 and best % 2 == 1):
            best, best_d = k, d
    return best


def e4m3_encode(x: float) -> int:
    """Round x to e4m3fn: nearest finite value, ties to even, saturating at +-448;
    NaN -> 0x7F; the sign bit is the sign of x (so -0.0 and small negatives give 0x80)."""
    if math.isnan(x):
        return 0x7F
    sign = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    return sign | _nearest_even(abs(x), E4M3_GRID)


def e2m1_encode(y: float) -> int:
    """Round y to E2M1: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to even, saturating at
    +-6; the sign bit is the sign of y.  (NaN never reaches here: the block quantizer
    handles NaN blocks first.)"""
    sign = 0x8 if math.copysign(1.0, y) < 0 else 0x0
    return sign | _nearest_even(abs(y), E2M1_GRID)


# ---- table-driven vectorized forms (same definitions, used on arrays) ----

E4M3_TABLE = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)
E2M1_TABLE = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)


def e4m3_decode_np(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode_np(codes: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.uint8) & 0xF]


def bf16_round_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest, ties to even (NaN stays a quiet NaN)."""
    b = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    r = ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x32, dtype=np.float32))
    r[nan] = ((b[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

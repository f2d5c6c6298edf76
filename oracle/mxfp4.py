"""MXFP4 codec in float64: E2M1 elements with a shared E8M0 scale per block of
32.  TEST INFRASTRUCTURE ONLY.

The oracle is a checker: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
path.

The SageAttention3 synthesis page names MXFP4, the OCP Microscaling format,
as the 4-bit format AMD's MI350-class GPUs support (Limitations: "NVFP4 vs
MXFP4", CosSim 98.37 % against NVFP4's 99.52 %).  The pages give no more of
it; what follows is that standard's definition:
  - element E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit, no
    infinities or NaN; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  - a block of 32 elements shares one E8M0 scale 2^e (code e + 127; no sign,
    no mantissa);
  - the scale of a block is 2^(floor(log2(amax)) - 2), 2 being the largest
    exponent of E2M1 (6 = 1.5 * 2^2), so amax / scale lies in [4, 8);
  - an element is x / scale rounded to nearest, ties to the even code, and
    saturated to +-6.
Readings: an all-zero block gets the smallest scale code 0 (2^-127) and zero
codes (of the values' signs); exponents are clamped to E8M0's range
[-127, 127].
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
MX_BLOCK = 32
E8M0_BIAS = 127
# magnitude of codes 0..7 (bit 3 is the sign)
_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64."""
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * _MAG[c & 7]


def encode(x) -> np.ndarray:
    """float -> E2M1 code (uint8 0..15): nearest magnitude, ties to the even
    code, saturated to 6; the sign bit is copied, so a negative value that
    rounds to zero gives -0 (code 8), as in IEEE rounding."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E2M1_MAX)
    # the grid is 0.5-spaced below 2 (codes 0..4), 1-spaced to 4 (codes
    # 4..6) and one step of 2 to 6 (codes 6..7): round on each piece
    lo = np.rint(a * 2.0)                                # codes 0..4 where a <= 2
    mid = 4.0 + np.rint(a - 2.0)                         # codes 4..6 where 2 <= a <= 4
    hi = 6.0 + np.rint((a - 4.0) / 2.0)                  # codes 6..7 where 4 <= a <= 6
    code = np.where(a <= 2.0, lo, np.where(a <= 4.0, mid, hi)).astype(np.int64)
    return (code | np.where(np.signbit(x), 8, 0)).astype(np.uint8)


def scale_exponent(amax) -> np.ndarray:
    """Shared exponent e of blocks with absolute maximum amax (int64)."""
    a = np.asarray(amax, dtype=np.float64)
    safe = np.where(a > 0, a, 1.0)
    e = np.floor(np.log2(safe)).astype(np.int64) - 2
    # np.log2 of an exact power of two is exact; guard the floor against a
    # value just below one
    e = np.where(np.exp2((e + 2).astype(np.float64)) > safe, e - 1, e)
    e = np.where(np.exp2((e + 3).astype(np.float64)) <= safe, e + 1, e)
    return np.clip(np.where(a > 0, e, -E8M0_BIAS), -E8M0_BIAS, E8M0_BIAS)


def quantize_blocks(x, axis: int = -1):
    """MX-quantize x in blocks of 32 consecutive elements along `axis` (the
    length must be a multiple of 32).  Returns (E2M1 codes uint8, shape of
    x; exponents int64, with `axis` shortened 32-fold)."""
    x = np.moveaxis(np.asarray(x, dtype=np.float64), axis, -1)
    n = x.shape[-1]
    assert n % MX_BLOCK == 0, n
    xb = x.reshape(*x.shape[:-1], n // MX_BLOCK, MX_BLOCK)
    e = scale_exponent(np.abs(xb).max(axis=-1))
    codes = encode(xb / np.exp2(e.astype(np.float64))[..., None])
    codes = np.moveaxis(codes.reshape(x.shape), -1, axis)
    return codes, np.moveaxis(e, -1, axis)


def dequantize_blocks(codes, e, axis: int = -1) -> np.ndarray:
    c = np.moveaxis(np.asarray(codes), axis, -1)
    ee = np.moveaxis(np.asarray(e, dtype=np.float64), axis, -1)
    v = decode(c).reshape(*c.shape[:-1], ee.shape[-1], MX_BLOCK) * np.exp2(ee)[..., None]
    return np.moveaxis(v.reshape(c.shape), -1, axis)

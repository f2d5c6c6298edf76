"""FP8 E4M3 (OCP "E4M3FN") codec in float64.  TEST INFRASTRUCTURE ONLY.

The oracle is a checker: only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg may import it.  It shares no code with the HIP
path.

The pages fix the format by its range: P is scaled by 448 "to the full range
of FP8 E4M3" (SageAttention2 detail page, Algorithm 1 and "Numerical
stability tricks", item 2; the SageAttention3 synthesis page gives the same
E4M3 maximum of 448).  448 is the largest finite value of the OCP E4M3
variant with no infinities (exponent bias 7, 3 mantissa bits, the all-ones
pattern S.1111.111 is NaN); that is the variant written here.  Rounding is
round-to-nearest-even with saturation to +-448 applied before rounding (the
reading recorded for the FP8 format: clamp, then RNE).

Everything is exact in float64: a value is scaled by a power of two onto an
integer grid and rounded with ``np.rint`` (half to even).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_EXP_BIAS = 7
_MIN_NORMAL_EXP = -6          # 2^-6 is the smallest normal
_MANT_BITS = 3


def decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS)
    nrm = (1.0 + m / 8.0) * np.exp2((e - _EXP_BIAS).astype(np.float64))
    val = np.where(e == 0, sub, nrm) * sign
    return np.where((e == 0xF) & (m == 0x7), np.nan, val)


def round_to_e4m3(x) -> np.ndarray:
    """Round float64 values onto the E4M3 grid: clamp to +-448, then RNE.

    Returns float64 values that are exactly representable in E4M3.
    """
    x = np.asarray(x, dtype=np.float64)
    s = np.sign(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # exponent of the binade holding a (frexp is exact): a = f * 2^e, f in [0.5, 1)
    _, e = np.frexp(a)
    e = np.maximum(e - 1, _MIN_NORMAL_EXP)          # subnormals share 2^-6's quantum
    quantum = np.ldexp(1.0, e - _MANT_BITS)
    r = np.rint(a / quantum) * quantum              # a/quantum is exact (power of 2)
    return s * r


def encode(x) -> np.ndarray:
    """float64 values -> uint8 E4M3 codes (clamp to +-448, then RNE).

    Negative values that round to zero keep the sign bit (0x80), as IEEE-style
    converters do; compare V codes by decoded value so that +-0 are equal.
    """
    x = np.asarray(x, dtype=np.float64)
    r = round_to_e4m3(x)
    neg = np.signbit(x)
    a = np.abs(r)
    _, e = np.frexp(a)
    e = e - 1
    is_sub = a < 2.0 ** _MIN_NORMAL_EXP
    m_sub = np.rint(a / 2.0 ** (_MIN_NORMAL_EXP - _MANT_BITS))
    # normal: a = (1 + m/8) 2^e
    m_nrm = np.rint((np.ldexp(a, -np.where(is_sub, 0, e)) - 1.0) * 8.0)
    e_fld = np.where(is_sub, 0, e + _EXP_BIAS)
    m_fld = np.where(is_sub, m_sub, m_nrm)
    code = (e_fld.astype(np.int64) << 3) | m_fld.astype(np.int64)
    code = np.where(a == 0, 0, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)

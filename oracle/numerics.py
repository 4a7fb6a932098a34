"""Element decodes for the oracle: OCP FP8 E4M3 (e4m3fn) and bf16.

Test infrastructure only (see the package docstring).

The pages name the expert format only as "FP8" with 128-wide scale blocks
(metrale ``fp8_moe_grouped.rs``, doc of ``fp8_grouped_tc_shape_ok``).  The
reading taken is the OCP 8-bit floating point E4M3 encoding ("e4m3fn"): one
sign bit, four exponent bits with bias 7, three mantissa bits; exponent field 0
encodes subnormals ``m/8 * 2**-6``; the all-ones exponent with all-ones mantissa
is NaN; there is no infinity, so the largest finite value is 448.

bf16 is the upper half of an IEEE binary32: widening is exact.
"""

from __future__ import annotations

import math

import numpy as np


def e4m3_value(code: int) -> float:
    """Value of one e4m3fn byte, from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return math.nan
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** (-6)
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def e4m3_table() -> np.ndarray:
    """All 256 code values as float64 (index = code)."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


_E4M3 = None


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    global _E4M3
    if _E4M3 is None:
        _E4M3 = e4m3_table()
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) exactly to float64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)

"""Element decodes for the oracle: OCP FP8 E4M3 (e4m3fn), OCP MXFP4 (E2M1
elements with E8M0 block scales) and bf16.

Test infrastructure only (see the package docstring).

The pages name the expert format only as "FP8" with 128-wide scale blocks
(metrale ``fp8_moe_grouped.rs``, doc of ``fp8_grouped_tc_shape_ok``).  The
reading taken is the OCP 8-bit floating point E4M3 encoding ("e4m3fn"): one
sign bit, four exponent bits with bias 7, three mantissa bits; exponent field 0
encodes subnormals ``m/8 * 2**-6``; the all-ones exponent with all-ones mantissa
is NaN; there is no infinity, so the largest finite value is 448.

The pages' 4-bit experts are NVFP4 (metrale ``forward_nvfp4_grouped_decode.rs``:
the grouped decode over 4-bit E2M1 experts with block scales).  gfx950's
native 4-bit block format is OCP microscaling MXFP4, the reading taken here:
E2M1 elements (one sign bit, two exponent bits with bias 1, one mantissa bit;
exponent field 0 encodes the subnormal ``m/2``; no infinity or NaN, largest
magnitude 6) sharing one E8M0 scale per 32 consecutive elements along the
depth (an unsigned exponent byte: ``2**(e - 127)``, 255 is NaN).

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


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code, from the bit fields."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    exp = (code >> 1) & 0x3
    man = code & 0x1
    if exp == 0:
        return sign * man * 0.5
    return sign * (1.0 + man / 2.0) * 2.0 ** (exp - 1)


def e2m1_table() -> np.ndarray:
    """All 16 code values as float64 (index = code)."""
    return np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)


def e8m0_value(byte: int) -> float:
    """Value of one E8M0 scale byte: 2**(e - 127), NaN for 255."""
    byte = int(byte) & 0xFF
    return math.nan if byte == 0xFF else 2.0 ** (byte - 127)


def mxfp4_decode(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Matrix [N, K] as float64 from packed codes [N, K/2] (two per byte, the
    lower nibble holding the even column) and E8M0 scales [N, K/32]: each
    element is its code's E2M1 value times the scale of its 32-column block."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, half = packed.shape
    K = 2 * half
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = packed & 0xF
    codes[:, 1::2] = packed >> 4
    vals = e2m1_table()[codes]
    sc = np.array([e8m0_value(b) for b in range(256)], dtype=np.float64)[np.asarray(scales, dtype=np.uint8)]
    assert sc.shape == (N, K // 32)
    return vals * np.repeat(sc, 32, axis=1)

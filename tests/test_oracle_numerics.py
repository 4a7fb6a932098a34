"""Pins of the oracle's element decodes: OCP e4m3fn and bf16.

The e4m3 table is checked against spot values fixed by the OCP definition and
against torch's float8_e4m3fn decode (an independent library routine); bf16
widening against torch's bfloat16 conversion over all 65536 patterns.
"""

import math

import numpy as np
import torch

import oracle
from oracle.numerics import e4m3_decode


def test_e4m3_spot_values():
    v = oracle.e4m3_value
    assert v(0x38) == 1.0
    assert v(0x7E) == 448.0
    assert v(0xFE) == -448.0
    assert v(0x08) == 2.0 ** -6
    assert v(0x01) == 2.0 ** -9
    assert v(0x07) == 7 * 2.0 ** -9
    assert v(0x00) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert math.isnan(v(0x7F)) and math.isnan(v(0xFF))
    assert v(0x40) == 2.0 and v(0x3C) == 1.5


def test_e4m3_table_matches_torch():
    t = oracle.e4m3_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(t), nan)
    assert np.array_equal(t[~nan], lib[~nan])
    assert np.array_equal(np.signbit(t[~nan]), np.signbit(lib[~nan]))


def test_e4m3_order_and_symmetry():
    t = oracle.e4m3_table()
    pos = t[0:0x7F]
    assert np.all(np.diff(pos) > 0)           # codes 0..0x7E strictly increasing
    assert np.array_equal(t[0x80:0xFF], -t[0:0x7F])
    assert np.nanmax(np.abs(t)) == 448.0
    assert int(np.isnan(t).sum()) == 2


def test_e4m3_decode_vectorised():
    codes = np.array([[0x38, 0x7E], [0x01, 0xC0]], dtype=np.uint8)
    assert np.array_equal(e4m3_decode(codes), np.array([[1.0, 448.0], [2.0 ** -9, -2.0]]))


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])


# ---------------------------------------------------------------- MXFP4 --

def test_e2m1_spot_values():
    """The OCP E2M1 values: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert oracle.e2m1_value(c) == want[c]
        assert oracle.e2m1_value(c | 8) == -want[c]
    assert math.copysign(1.0, oracle.e2m1_value(8)) == -1.0


def test_e2m1_equals_e4m3_with_rebiased_fields():
    """E2M1 (bias 1) is E4M3 (bias 7) with the exponent field raised by 6 and
    the mantissa bit moved to the top mantissa bit; the subnormal 0.5 is the
    e4m3 normal 2**-1.  Checked through the torch-pinned e4m3 decode."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e == 0 and m == 0:
            code = s << 7
        elif e == 0:
            code = (s << 7) | (6 << 3)
        else:
            code = (s << 7) | ((e + 6) << 3) | (m << 2)
        assert oracle.e2m1_value(c) == oracle.e4m3_value(code), c


def test_e8m0_matches_torch():
    got = np.array([oracle.e8m0_value(b) for b in range(256)])
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert oracle.e8m0_value(127) == 1.0 and oracle.e8m0_value(130) == 8.0 and math.isnan(oracle.e8m0_value(255))


def test_mxfp4_decode_layout_and_scale_locality():
    rng = np.random.default_rng(3)
    N, K = 4, 128
    packed = rng.integers(0, 256, size=(N, K // 2)).astype(np.uint8)
    scales = rng.integers(120, 135, size=(N, K // 32)).astype(np.uint8)
    w = oracle.mxfp4_decode(packed, scales)
    tab = oracle.e2m1_table()
    # lower nibble = even column, upper = odd, times the row's 32-column block scale
    for r, c in [(0, 0), (0, 1), (1, 31), (2, 32), (3, 127), (2, 64)]:
        code = (packed[r, c // 2] >> (4 * (c % 2))) & 0xF
        assert w[r, c] == tab[code] * 2.0 ** (int(scales[r, c // 32]) - 127)
    # one scale byte up by one doubles exactly its 32 elements and nothing else
    s2 = scales.copy()
    s2[1, 2] += 1
    w2 = oracle.mxfp4_decode(packed, s2)
    diff = w2 != w
    assert not diff[:, :64].any() and not diff[:, 96:].any() and not diff[[0, 2, 3]].any()
    assert np.array_equal(w2[1, 64:96], 2 * w[1, 64:96])
    # one nibble changes one element
    p2 = packed.copy()
    p2[3, 5] ^= 0x30
    d = oracle.mxfp4_decode(p2, scales) != w
    assert d.sum() <= 1 and not d[:, :11].any() and not d[:, 12:].any()

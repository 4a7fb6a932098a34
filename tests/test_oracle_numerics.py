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

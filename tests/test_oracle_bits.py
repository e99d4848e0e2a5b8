"""Pins for the oracle's input decoding (oracle/bits.py): bfloat16 bit
patterns whose values the format fixes (sign, 8-bit exponent with bias 127,
7 stored fraction bits)."""

import math

import numpy as np

from oracle import bits


def test_bf16_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x0001, 0x7F80, 0x3F81, 0x4300], dtype=np.uint16)
    vals = bits.bf16_to_f64(pats)
    assert vals[0] == 1.0 and vals[1] == -2.0 and vals[2] == 3.140625
    assert vals[3] == 0.0 and math.copysign(1.0, vals[4]) == -1.0
    assert vals[5] == 2.0 ** -133 and math.isinf(vals[6])
    assert vals[7] == 1.0 + 2.0 ** -7 and vals[8] == 128.0


def test_to_f64_passes_float_through():
    x = np.array([1.5, -0.25], dtype=np.float32)
    assert bits.to_f64(x).tolist() == [1.5, -0.25]


def test_to_f64_reads_uint16_as_bf16_bits():
    """uint16 arrays are bf16 bit patterns (0x3F80 is 1.0, 0xC040 is -3.0);
    float arrays widen as they are."""
    got = bits.to_f64(np.array([0x3F80, 0xC040, 0x0000], dtype=np.uint16))
    np.testing.assert_array_equal(got, [1.0, -3.0, 0.0])
    np.testing.assert_array_equal(bits.to_f64(np.array([0.1], dtype=np.float32)), [float(np.float32(0.1))])

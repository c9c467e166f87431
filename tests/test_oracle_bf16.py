"""Pins for the exact bfloat16 decoder of the oracle: known bit patterns from
the IEEE binary32 layout (bfloat16 keeps its sign, its 8 exponent bits and the
top 7 fraction bits), and a round trip through torch's own bfloat16 type."""
import math

import numpy as np
import pytest

from oracle.bf16 import bf16_to_f64, to_f64


@pytest.mark.parametrize("bits,value", [
    (0x0000, 0.0),
    (0x3F80, 1.0),                  # exponent 127, fraction 0
    (0xBF80, -1.0),                 # sign bit
    (0x4000, 2.0),
    (0x3F00, 0.5),
    (0x4049, 3.140625),             # 1.1001001b x 2^1
    (0x3F81, 1.0 + 2.0 ** -7),      # lowest fraction bit = one ulp above 1
    (0x7F7F, (2.0 - 2.0 ** -7) * 2.0 ** 127),   # largest finite
    (0x0080, 2.0 ** -126),          # smallest normal
    (0x0001, 2.0 ** -133),          # smallest subnormal: 2^-126 x 2^-7
    (0x807F, -(1.0 - 2.0 ** -7) * 2.0 ** -126),  # largest negative subnormal
])
def test_known_bit_patterns(bits, value):
    got = bf16_to_f64(np.array([bits], dtype=np.uint16))[0]
    assert got == value


def test_signed_zero_infinities_and_nan():
    got = bf16_to_f64(np.array([0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1], dtype=np.uint16))
    assert got[0] == 0.0 and math.copysign(1.0, got[0]) < 0
    assert got[1] == math.inf and got[2] == -math.inf
    assert np.isnan(got[3]) and np.isnan(got[4])


def test_every_pattern_round_trips_through_torch_bfloat16():
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    ref = t.to(torch.float64).numpy()
    got = bf16_to_f64(bits)
    finite = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~finite)
    assert np.array_equal(got[finite], ref[finite])
    # the sign of zero survives too
    assert np.array_equal(np.signbit(got[finite]), np.signbit(ref[finite]))
    # f32 storage decodes unchanged
    x = np.array([1.5, -2.25e-30, 3.0e38], dtype=np.float32)
    assert np.array_equal(to_f64(x, "f32"), x.astype(np.float64))

"""Pins for the oracle's bf16 bit helpers: hand-computed bit patterns and
PyTorch's float32 -> bfloat16 conversion (a library routine, round to
nearest even)."""

import math

import numpy as np
import pytest
import torch

from oracle import bf16


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xBF80, -1.0), (0x4000, 2.0), (0x3F00, 0.5),
    (0x4049, 3.140625), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126),
    (0x7F7F, (2 - 2.0 ** -7) * 2.0 ** 127), (0x0000, 0.0),
])
def test_to_f64_known(bits, value):
    assert bf16.to_f64(np.array([bits], np.uint16))[0] == value


def test_to_f64_specials():
    x = bf16.to_f64(np.array([0x7F80, 0xFF80, 0x8000, 0x7FC1], np.uint16))
    assert x[0] == math.inf and x[1] == -math.inf
    assert x[2] == 0.0 and math.copysign(1.0, x[2]) == -1.0
    assert math.isnan(x[3])


@pytest.mark.parametrize("value,bits", [
    (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie -> even (down)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie -> even (up)
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
    (1.0 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),    # just below the tie
    (2.0 - 2.0 ** -9, 0x4000),                 # carry into the exponent
    (-(1.0 + 3 * 2.0 ** -8), 0xBF82),          # sign is kept
    (3.4e38, 0x7F80),                          # beyond max + half ulp -> inf
    (2.0 ** -133, 0x0001),                     # smallest subnormal
])
def test_from_f64_rounding(value, bits):
    assert int(bf16.from_f64(np.array([value]))[0]) == bits


def test_from_f64_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        rng.integers(-(2 ** 31), 2 ** 31, 50000).astype(np.int32).view(np.float32),
    ])
    x = x[np.isfinite(x)]
    ours = bf16.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_round_trip_exact():
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    finite = bits[exp != 0xFF]
    assert np.array_equal(bf16.from_f64(bf16.to_f64(finite)), finite)

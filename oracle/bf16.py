"""bf16 bit helpers for the oracle (test infrastructure only).

bf16 is the upper 16 bits of an IEEE-754 binary32.  numpy has no bf16 dtype in
this environment, so bf16 tensors are held as ``uint16`` bit patterns.

* ``to_f64``: exact widening (every bf16 value is a binary32 value, and every
  binary32 value is a binary64 value).
* ``from_f64``: rounding to bf16, round-to-nearest, ties-to-even, via binary32
  (first to the nearest binary32, then to bf16 from the binary32 bits).  The
  output precision is bf16 with fp32 accumulation upstream; the double
  rounding through binary32 is stated here and matches what a device that
  accumulates in fp32 does.

Pinned by ``tests/test_oracle_bf16.py`` against hand-computed bit patterns
(ties, carries into the exponent, signed zero, infinities) and against
PyTorch's own float32 -> bfloat16 conversion (a library routine).
"""

import numpy as np


def to_f64(u16):
    """Widen bf16 bit patterns (uint16 array) to float64, exactly."""
    u16 = np.asarray(u16, dtype=np.uint16)
    u32 = u16.astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def f32_to_bf16(f32):
    """Round float32 values to bf16 bits, nearest with ties to even.

    Adding 0x7FFF plus the lowest kept bit and truncating is the standard
    integer form of round-half-to-even on the dropped 16 bits.  NaN inputs are
    mapped to a quiet NaN so the addition cannot turn them into infinities.
    """
    f32 = np.ascontiguousarray(f32, dtype=np.float32)
    u32 = f32.view(np.uint32).astype(np.uint64)
    lsb = (u32 >> np.uint64(16)) & np.uint64(1)
    r = ((u32 + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f32)
    if nan.any():
        r = np.where(nan, ((u32 >> np.uint64(16)).astype(np.uint16) | np.uint16(0x0040)), r)
    return r.astype(np.uint16)


def from_f64(x):
    """Round float64 values to bf16 bits (via binary32, ties to even)."""
    return f32_to_bf16(np.asarray(x, dtype=np.float64).astype(np.float32))

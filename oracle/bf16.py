"""Oracle O6: fp32 -> bf16 round-to-nearest, ties-to-even, from its definition.
TEST INFRASTRUCTURE ONLY.

The bf16 param is the 2-byte weight that sits beside the fp32 master
([Megatron DP] "朴素 DP 的致命浪费" table: bf16 weight 2 B, fp32 master 4 B);
after the partition update the new master is written back to it.  Rounding is
IEEE round-to-nearest-even onto the bf16 grid (8 exponent bits, 7 stored
mantissa bits); overflow goes to infinity as IEEE specifies (the value is
rounded as if the exponent were unbounded, and 2^128 becomes inf); NaN stays
NaN (quiet, sign and top payload bits kept).

Written from the definition, not as a bit trick: for each fp32 value take the
two neighbouring bf16 magnitudes (toward zero and away from zero), measure both
distances exactly in float64, pick the nearer, and on a tie the one whose last
mantissa bit is 0.
"""

import numpy as np


def _bf16_magnitude_value(mag16):
    """float64 value of a non-negative bf16 magnitude pattern (uint32 array),
    with the pattern 0x7F80 read as 2^128 (the unbounded-exponent successor of
    the largest finite bf16)."""
    full = (mag16.astype(np.uint32) << np.uint32(16)).view(np.float32)
    with np.errstate(invalid="ignore"):
        val = full.astype(np.float64)
    return np.where(mag16 == 0x7F80, 2.0 ** 128, val)


def bf16_rne_oracle(x):
    """float32 array -> uint16 array of bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = (bits >> np.uint32(31)).astype(np.uint32)
    mag = bits & np.uint32(0x7FFFFFFF)
    is_nan = mag > np.uint32(0x7F800000)
    is_inf = mag == np.uint32(0x7F800000)

    lo = mag >> np.uint32(16)               # toward zero
    hi = lo + np.uint32(1)                  # away from zero
    with np.errstate(invalid="ignore"):
        absx = np.abs(x.astype(np.float64))
    d_lo = absx - _bf16_magnitude_value(lo)
    d_hi = _bf16_magnitude_value(np.minimum(hi, np.uint32(0x7F80))) - absx
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    exact = (mag & np.uint32(0xFFFF)) == 0
    rounded = np.where(exact, lo, np.where(pick_hi, hi, lo))

    out = (sign << np.uint32(15)) | rounded
    out = np.where(is_inf, (sign << np.uint32(15)) | np.uint32(0x7F80), out)
    nan_out = (bits >> np.uint32(16)) | np.uint32(0x0040)
    out = np.where(is_nan, nan_out, out)
    return out.astype(np.uint16)

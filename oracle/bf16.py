"""bf16 rounding (oracle; test infrastructure).

Round-to-nearest-even of binary32 values to bfloat16 (the top 16 bits of a
binary32), written from the definition.  Pinned against torch's CPU
conversion in tests/test_oracle_step.py.
"""

import numpy as np


def bf16_round(x):
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 patterns.

    Written from the definition: the two bf16 neighbours of |x| are the value
    with the low 16 bits cleared and the next bf16 above it (for the largest
    finite bf16 that is 2^128, which stands for infinity); both distances are
    exact in float64 and the nearer one wins, the one with an even mantissa on
    a tie.
    """
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    sign = (bits >> np.uint32(16)) & np.uint32(0x8000)
    mag = bits & np.uint32(0x7FFFFFFF)
    lo_bits = mag & np.uint32(0xFFFF0000)
    hi_bits = lo_bits + np.uint32(0x10000)
    is_top = hi_bits == np.uint32(0x7F800000)
    with np.errstate(over="ignore", invalid="ignore"):
        lo = lo_bits.view(np.float32).astype(np.float64)
        hi = np.where(is_top, 2.0 ** 128, hi_bits.view(np.float32).astype(np.float64))
        a = mag.view(np.float32).astype(np.float64)
        d_lo = a - lo
        d_hi = hi - a
    lo_odd = ((lo_bits >> np.uint32(16)) & np.uint32(1)) == 1
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & lo_odd)
    out = np.where(take_hi, hi_bits >> np.uint32(16), lo_bits >> np.uint32(16))
    is_inf = mag == np.uint32(0x7F800000)
    is_nan = mag > np.uint32(0x7F800000)
    out = np.where(is_inf, np.uint32(0x7F80), out)
    out = np.where(is_nan, np.uint32(0x7FC0), out)
    return (out | sign).astype(np.uint16)

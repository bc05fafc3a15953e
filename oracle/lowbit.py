"""A low-bit KV cache format for the oracle: 8-bit floating point E4M3 as
defined by the OCP 8-bit floating point specification (the FN variant: no
infinities, one NaN pattern per sign).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[FD] paper summary page, 未来方向 item (3): fused kernels over a low-bit KV
cache are named as a direction to explore.  The pages fix no format; the
reading taken here: K and V are stored as E4M3 codes with a unit scale,
rounded to nearest with ties to even, magnitudes beyond the largest finite
value (448) saturating to it; attention reads the decoded values.

Code layout: bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa.
Exponent 0 is subnormal (m * 2^-9); exponent 15 with mantissa 7 is NaN;
every other pattern is normal, 2^(e-7) * (1 + m/8).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values (the format's definition, term by term)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m * 2.0 ** -9
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# the 127 non-negative finite values, in code order 0x00 .. 0x7e (increasing)
_TABLE = e4m3_decode(np.arange(0x7F))


def e4m3_encode(x) -> np.ndarray:
    """float values -> uint8 codes: the nearest finite value, ties to the
    even code (mantissa bit 0 clear), saturating at +-448; the sign bit is
    the input's sign bit (so a negative value that rounds to zero gives 0x80).
    Inputs must not be NaN."""
    a = np.asarray(x, dtype=np.float64)
    if np.isnan(a).any():
        raise ValueError("NaN input")
    mag = np.minimum(np.abs(a), E4M3_MAX)
    lo = np.clip(np.searchsorted(_TABLE, mag, side="right") - 1, 0, len(_TABLE) - 1)
    hi = np.minimum(lo + 1, len(_TABLE) - 1)
    d_lo = mag - _TABLE[lo]
    d_hi = _TABLE[hi] - mag
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (lo % 2 == 1))
    code = np.where(take_hi, hi, lo).astype(np.int64)
    code = code | np.where(np.signbit(a), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_round(x) -> np.ndarray:
    """The value a cache entry holds after storing x: decode(encode(x))."""
    return e4m3_decode(e4m3_encode(x))

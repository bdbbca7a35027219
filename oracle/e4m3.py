"""OCP 8-bit floating point, E4M3FN variant (oracle; test infrastructure only).

The LampAttention abstract evaluates key-query products and exponentials "in
8-bit formats"; the format used here is the OCP E4M3 encoding as implemented
by gfx950 hardware: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits,
subnormals, no infinities, a single NaN pattern per sign (S.1111.111), largest
finite magnitude 448.

Encoding is round-to-nearest, ties to the even code, and saturating (values
beyond 448 in magnitude encode as +-448).  The sign of zero is kept: a negative
input that rounds to zero encodes as 0x80.
"""
import numpy as np

E4M3_MAX = 448.0
NAN_MAG = 0x7F


def decode(codes):
    """Value of each E4M3FN code (uint8 array) as float64; NaN for 0x7F/0xFF."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = m.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    mag = np.where(e == 0, sub, nrm)
    mag = np.where((c & 0x7F) == NAN_MAG, np.nan, mag)
    return sign * mag


# the 127 finite non-negative magnitudes, indexed by code 0x00..0x7E
_MAGS = decode(np.arange(0, NAN_MAG, dtype=np.uint8))


def encode(x):
    """Round float64 values to E4M3FN codes (RNE, saturating, signed zero)."""
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        raise ValueError("e4m3.encode: NaN input")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_MAGS, a, side="left")          # first magnitude >= a
    hi = np.minimum(hi, NAN_MAG - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _MAGS[lo]
    d_hi = _MAGS[hi] - a
    # exact hit: hi is the value itself
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    neg = np.signbit(x)
    code = np.where(neg, code | 0x80, code)
    return code.astype(np.uint8)


def round_to_e4m3(x):
    """x rounded to the nearest E4M3FN value (RNE, saturating), as float64."""
    return decode(encode(x))


def rounding_boundaries():
    """Sorted non-negative magnitudes at which RNE rounding to E4M3 changes code.

    These are the midpoints between consecutive finite magnitudes.  Magnitudes
    above 448 saturate, so there is no boundary there.
    """
    return 0.5 * (_MAGS[1:] + _MAGS[:-1])

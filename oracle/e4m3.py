"""The e4m3 8-bit floating-point format (oracle; test infrastructure only).

[P2] "Fused attention kernel", Variants / 8-bit forward pass (FP8, Hopper): the
8-bit path stores Q, K and V in the e4m3 format.  [P1] "How it gets verified":
Q, K, V in E4M3.

The pages name the format but do not define it.  This module takes the OCP
8-bit float definition of e4m3 (the "fn" variant, which the MI355X converts
produce): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals
when the exponent field is 0, no infinities, and NaN only for the codes 0x7F
and 0xFF.  The largest finite magnitude is 1.75 * 2**8 = 448.

Encoding rule (a reading; the pages do not fix it): round to the nearest
representable value, ties to an even mantissa; saturate magnitudes above 448
to 448 (never produce NaN); keep the sign of zero and of values that round to
zero.  Inputs must be finite.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6          # smallest normal value is 2**-6
_MANT_BITS = 3


def decode(codes):
    """Value of each e4m3 code as float64 (closed form); 0x7F/0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    subnormal = m * np.ldexp(1.0, -9)
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def encode(values):
    """e4m3 code (uint8) of each finite float: round-to-nearest-even, saturate to +-448.

    Works in float64, where every step below is exact for float32 or float64
    inputs: the quantum of the binade is a power of two, so ``a / quantum`` is
    exact and ``np.rint`` rounds half to even.
    """
    v = np.asarray(values, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3 encode: non-finite input is outside the contract")
    sign = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    # binade exponent floor(log2 a), clamped to the subnormal range
    _, fexp = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(fexp - 1, _MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - _MANT_BITS)
    r = np.rint(a / quantum) * quantum          # nearest, ties to even
    r = np.minimum(r, E4M3_MAX)                 # saturate (satfinite)
    # bits of the rounded magnitude r
    is_sub = r < 2.0 ** _MIN_NORMAL_EXP
    m_sub = np.rint(r / 2.0 ** -9).astype(np.int64)
    _, rexp = np.frexp(np.where(r > 0, r, 1.0))
    re = rexp - 1
    m_norm = np.rint((r / np.ldexp(1.0, re) - 1.0) * 8.0).astype(np.int64)
    mag = np.where(is_sub, m_sub, ((re + 7) << 3) | m_norm)
    return ((sign << 7) | mag).astype(np.uint8)


def all_finite_codes():
    """The 254 non-NaN codes as a uint8 array."""
    c = np.arange(256, dtype=np.int64)
    return c[(c & 0x7F) != 0x7F].astype(np.uint8)

"""Schraudolph's bit-level exponential, base 2, float32 (oracle; test infrastructure only).

Method: N. N. Schraudolph, "A fast, compact approximation of the exponential
function", Neural Computation 11(4), 1999.  An IEEE float whose exponent field
holds floor(y) + bias and whose mantissa holds the fractional part of y,
linearly, has the value 2^floor(y) * (1 + frac(y)): a piecewise-linear
interpolation of 2^y between powers of two.  Writing the integer
floor(2^23 (y + 127)) into the 32 bits of a float32 builds exactly that number
(for y in the normal range).  Schraudolph shifts y by a constant to centre the
error; his constant is 60801 in units of 2^-20 of the exponent (the 2^20 scale
belongs to his double-precision formulation; expressed in exponent units it is
sigma = 60801 / 2^20 for any width).  FLAMIA ("FLAMIA: FLAsh MIcroscaling
Attention", 4.4 Bit-Level Exponentials at Inference) evaluates this
approximation for the probabilities of attention at inference.

Readings taken here:
  * working precision: the method forms its integer from a floating-point
    expression, A y + B, evaluated in the working precision (his formulation:
    double; here float32).  So 2^23 (x + 127 - sigma) is rounded to float32
    (round to nearest even) before it is floored.  Its magnitude is about 2^30,
    so this rounding moves the integer by up to 32 (of 2^23 per octave), a
    relative change of the result below 2^-17: small, but enough to move an
    e4m3 rounding of the result across a boundary now and then, so the
    oracle keeps it.
  * range ends (the method is stated for the normal range): the integer is
    saturated to [0, 2^32 - 1], so inputs below -127 + sigma give +0 (and -inf
    gives +0), as the unsigned float-to-integer conversion of the GPU does
    (round toward zero, saturating).
"""

import numpy as np

SIGMA = 60801.0 / 2.0 ** 20


def schraudolph_exp2(x):
    """2^x approximated bit-wise: the float32 with bits floor(fl32(2^23 (x + 127 - SIGMA))).

    x: float64 array; returns float64 values of the resulting float32 numbers.
    Relative error in [2^-SIGMA - 1, (1/ln 2) 2^(1 - 1/ln 2 - SIGMA) - 1] (about
    -3.9% .. +2.0%), widened by the float32 rounding of the argument (< 2^-17).
    """
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        arg = ((x + (127.0 - SIGMA)) * 2.0 ** 23).astype(np.float32)   # the float32 argument
        v = np.floor(arg.astype(np.float64))
    v = np.where(np.isnan(v), 0.0, np.clip(v, 0.0, 2.0 ** 32 - 1))
    return v.astype(np.uint64).astype(np.uint32).view(np.float32).astype(np.float64)

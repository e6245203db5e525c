"""Sylvester Hadamard matrix and its fast transform (oracle; test infrastructure only).

[P2] "Fused attention kernel", Variants / 8-bit forward pass: Q and K are
rotated by the same orthogonal transform, a random +-1 diagonal followed by a
Hadamard matrix; an orthogonal transform applied to both leaves every dot
product q . k, and so the attention output, unchanged in exact arithmetic,
while it spreads a large channel over all channels.

Readings taken here (the pages do not fix them):
  * The Hadamard matrix is Sylvester's, in natural order:
    H_1 = [1],  H_2n = [[H_n, H_n], [H_n, -H_n]], so H_d H_d^T = d I.
  * The kernel applies the UNnormalised H_d (entries +-1, exact); the missing
    1/sqrt(d) on each of Q and K becomes one exact factor 1/d on the scores.
  * For bit-exact float32 emulation the transform is evaluated as the fast
    Walsh-Hadamard transform with butterfly stages h = 1, 2, 4, ..., d/2 in that
    order; each stage replaces (y_i, y_{i+h}) for every i with (i & h) == 0 by
    (y_i + y_{i+h}, y_i - y_{i+h}), each rounded to float32.
"""

import numpy as np


def sylvester(d):
    """Sylvester Hadamard matrix H_d (int64), d a power of two, by its recursive definition."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1), dtype=np.int64)
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def fwht_f32(y):
    """y @ H_d along the last axis, in float32, stage order h = 1, 2, ..., d/2."""
    y = np.array(y, dtype=np.float32, copy=True)
    d = y.shape[-1]
    if d < 1 or d & (d - 1):
        raise ValueError("last dim must be a power of two")
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        s = a + b            # float32 + float32 -> float32, round to nearest even
        t = a - b
        y = np.stack([s, t], axis=-2).reshape(lead + (d,))
        h *= 2
    return y


def fwht_f64(y):
    """Same transform in float64 (for tests of the float32 rounding error)."""
    y = np.array(y, dtype=np.float64, copy=True)
    d = y.shape[-1]
    lead = y.shape[:-1]
    h = 1
    while h < d:
        z = y.reshape(lead + (d // (2 * h), 2, h))
        a = z[..., 0, :]
        b = z[..., 1, :]
        y = np.stack([a + b, a - b], axis=-2).reshape(lead + (d,))
        h *= 2
    return y

"""Philox4x32-10 and the random sign diagonal (oracle; test infrastructure only).

[P2] "Fused attention kernel", Variants / 8-bit forward pass: incoherent
processing multiplies Q and K by an orthogonal matrix built from a random sign
diagonal and a Hadamard matrix.  The pages do not say how the signs are drawn.

Reading taken here: the signs come from the counter-based generator
Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
as 1, 2, 3", SC 2011), written from that published definition:
  * one round maps counter (x0, x1, x2, x3) and key (k0, k1) to
      (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0))
    with M0 = 0xD2511F53, M1 = 0xCD9E8D57 (32x32 -> 64-bit products);
  * between rounds the key is bumped by the Weyl constants
    (0x9E3779B9, 0xBB67AE85); ten rounds in all.
The sign vector for a call with 64-bit ``seed`` uses ONE block:
counter = (0, 0, 0, 0), key = (seed mod 2**32, seed >> 32).  Its four 32-bit
words, concatenated little-end first, give 128 bits; channel c gets
sigma_c = -1 if bit c is set, else +1.  One sign vector serves every batch and
head, and the same vector rotates Q and K (required for the rotation to
cancel in Q K^T).  Head dims up to 128 are covered.
"""

import numpy as np

_M0 = 0xD2511F53
_M1 = 0xCD9E8D57
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = 0xFFFFFFFF


def philox4x32_10(counter, key):
    """One Philox4x32-10 block: 4 counter words, 2 key words -> 4 uint32 words."""
    x = [int(w) & _MASK for w in counter]
    k = [int(w) & _MASK for w in key]
    for rnd in range(10):
        if rnd > 0:
            k[0] = (k[0] + _W0) & _MASK
            k[1] = (k[1] + _W1) & _MASK
        p0 = _M0 * x[0]
        p1 = _M1 * x[2]
        x = [(p1 >> 32) ^ x[1] ^ k[0], p1 & _MASK, (p0 >> 32) ^ x[3] ^ k[1], p0 & _MASK]
    return x


def sign_vector(seed, d):
    """sigma in {+1, -1}^d (float32) for a call with 64-bit ``seed``; d <= 128."""
    if not 0 < d <= 128:
        raise ValueError("sign_vector covers head dims 1..128")
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    words = philox4x32_10((0, 0, 0, 0), (seed & _MASK, seed >> 32))
    bits = [(words[c // 32] >> (c % 32)) & 1 for c in range(d)]
    return np.where(np.array(bits, dtype=np.int64) == 1, -1.0, 1.0).astype(np.float32)

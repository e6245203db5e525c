"""Rotate + per-block scale + e4m3 encode of Q, K, V (oracle; test infrastructure only).

[P2] "Fused attention kernel", Variants / 8-bit forward pass (FP8, Hopper):
  * scales are chosen per block, separately for Q, K and V, rather than once
    for a whole tensor;
  * before Q and K (never V) are quantised they are rotated by one orthogonal
    transform: a random +-1 diagonal followed by a Hadamard matrix.
[P3] FLAMIA, 4.3 Ablation Study: quantisation fused into one launch, and score
scales folded together (the 1/d of the unnormalised Hadamard and the block
descales fold into the score scale on the attention side).

The pages leave the block shape, the scale formula and the rounding open.
Readings taken here:
  * a block is ``scale_block`` consecutive tokens of one (batch, head) times all
    d channels; the last block of a sequence may be short and its maximum is
    taken over its valid tokens only;
  * with y the (rotated) float32 block and a = max |y| over the block:
      inv = fl32(448 / a),  descale = fl32(a / 448)   (correctly rounded float32
      division); a block of zeros gets inv = descale = 1;
  * code = e4m3(fl32(y * inv)) with the encoder of ``oracle.e4m3``;
  * rotation: y = x * sigma (exact), then the float32 fast Walsh-Hadamard
    transform of ``oracle.hadamard`` (unnormalised, stage order fixed).
  * V's blocks take the power-of-two form below in every mode: an e4m3 code
    has the same relative precision at any power-of-two scale, and such a
    scale is applied exactly inside the matrix core that forms P V, so P
    need not carry V's scale (the kernel then keeps P away from e4m3's
    subnormal range).
Dequantised value: e4m3_value(code) * descale.

Power-of-two (microscaling, E8M0) scales, the option ``pow2=True`` ([P3]
FLAMIA, 2 Background: MX formats give each block of low-bit codes one shared
scale, applied by block-scaled matrix units; the MX blocks there are 32
elements, which ``group=32`` gives: one scale per scale_block tokens x 32
channels).  The pages do not fix how the
exponent is chosen; the reading taken is the power-of-two form of the scale
above that never saturates: descale = 2^e with e the smallest integer such
that a <= 448 * 2^e, clamped to the E8M0 range [-127, 127]; inv = 2^-e; a block
of zeros gets 2^0.  (The scale rule of the OCP MX specification,
2^(floor(log2 a) - 8), would clip the block maximum by up to 12.5%.)

Everything below is float32 numpy arithmetic, which rounds every operation to
nearest even, so the result is the bit pattern the specification defines.
"""

import numpy as np

from . import e4m3
from .hadamard import fwht_f32
from .philox import sign_vector

_F448 = np.float32(448.0)


def num_blocks(n, scale_block):
    return -(-n // scale_block)


def rotate(x, signs):
    """x @ diag(signs) @ H_d along the last axis, float32 (signs exact +-1)."""
    y = np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    return fwht_f32(y)


def pow2_exponent(a):
    """Smallest integer e with a <= 448 * 2^e (a float32 >= 0), clamped to [-127, 127]; 0 for a = 0.

    Evaluated exactly: 448 * 2^e is exact in float64 over this range.
    """
    a = np.asarray(a, dtype=np.float64)
    _, ex = np.frexp(np.where(a > 0, a / 448.0, 1.0))   # a/448 = m 2^ex, m in [0.5, 1): exact for float32 a
    e = ex - 1                                           # 2^(ex-1) <= a/448 < 2^ex
    e = np.where(a <= 448.0 * np.exp2(e), e, e + 1)      # only exact powers of two stay at ex - 1
    e = np.where(a > 0, e, 0)
    return np.clip(e, -127, 127).astype(np.int64)


def quantize_tensor(x, scale_block, signs=None, pow2=False, group=None):
    """One tensor [..., N, d] -> (codes uint8 [..., N, d], descale float32).

    ``signs`` (float32 +-1 of length d) turns the rotation on; None leaves x unrotated.
    ``pow2`` selects the power-of-two (E8M0) block scales.  ``group`` (a divisor
    of d, power-of-two scales only) gives every block one scale per ``group``
    consecutive channels instead of one for all d: descale [..., nblk, d / group];
    otherwise descale [..., nblk].
    """
    y = np.asarray(x, dtype=np.float32)
    if signs is not None:
        y = rotate(y, signs)
    n, d = y.shape[-2], y.shape[-1]
    if group is not None and (not pow2 or d % group):
        raise ValueError("channel groups need power-of-two scales and must divide d")
    g = d if group is None else group
    nb = num_blocks(n, scale_block)
    lead = y.shape[:-2]
    amax = np.empty(lead + (nb, d // g), dtype=np.float32)
    for blk in range(nb):
        rows = y[..., blk * scale_block:min(n, (blk + 1) * scale_block), :]
        rows = rows.reshape(rows.shape[:-1] + (d // g, g))
        amax[..., blk, :] = np.abs(rows).max(axis=(-3, -1))
    zero = amax == 0
    if pow2:
        e = pow2_exponent(amax)
        inv = np.exp2(-e).astype(np.float32)             # exact: 2^-127 .. 2^127 are float32 values
        descale = np.exp2(e).astype(np.float32)
    else:
        with np.errstate(divide="ignore", invalid="ignore"):
            inv = np.where(zero, np.float32(1.0), _F448 / amax).astype(np.float32)
            descale = np.where(zero, np.float32(1.0), amax / _F448).astype(np.float32)
    inv_rows = np.repeat(inv, scale_block, axis=-2)[..., :n, :]          # [..., n, d / g]
    v = y * np.repeat(inv_rows, g, axis=-1)     # float32 product, round to nearest even
    return e4m3.encode(v), (descale if group is not None else descale[..., 0])


def quantize_qkv(q, k, v, scale_block, hadamard, seed, pow2=False, group=None):
    """The full pre-processing of one attention call.

    Returns (q8, k8, v8, q_descale, k_descale, v_descale).  Q and K share one
    sign vector drawn from ``seed``; V is never rotated.  V's blocks always
    take power-of-two scales (the product with P applies them exactly);
    ``pow2`` gives Q and K power-of-two scales too; ``group`` (with pow2)
    gives all three one scale per ``group`` channels of a block.
    """
    d = np.shape(q)[-1]
    signs = sign_vector(seed, d) if hadamard else None
    q8, qd = quantize_tensor(q, scale_block, signs, pow2, group)
    k8, kd = quantize_tensor(k, scale_block, signs, pow2, group)
    v8, vd = quantize_tensor(v, scale_block, None, True, group)
    return q8, k8, v8, qd, kd, vd


def dequantize(codes, descale, scale_block):
    """float64 value of each code times its block's descale (descale [..., nblk]
    or, with channel groups, [..., nblk, d / group])."""
    vals = e4m3.decode(codes)
    n, d = vals.shape[-2], vals.shape[-1]
    ds = np.asarray(descale, dtype=np.float64)
    if ds.ndim == vals.ndim:                     # channel groups
        ds = np.repeat(np.repeat(ds, scale_block, axis=-2)[..., :n, :], d // ds.shape[-1], axis=-1)
        return vals * ds
    ds = np.repeat(ds, scale_block, axis=-1)[..., :n]
    return vals * ds[..., None]

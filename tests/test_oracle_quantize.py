"""Pins of the oracle's rotate + block-scale + e4m3 quantiser.

Hand-derived worked examples (tests/golden), the scale-invariance and
error-bound properties of a block-scaled float format, block causality, and
the cancellation of the rotation in Q K^T.
"""

import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import e4m3, quantize
from oracle.philox import sign_vector

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quantize_worked_example.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_worked_examples(ex):
    x = np.array(ex["x"], dtype=np.float32)[None, None]
    signs = None if ex["signs"] is None else np.array(ex["signs"], dtype=np.float32)
    codes, descale = quantize.quantize_tensor(x, ex["scale_block"], signs)
    assert codes[0, 0].tolist() == ex["codes"]
    amax = np.array(ex["amax"], dtype=np.float32)
    assert np.array_equal(descale[0, 0], amax / np.float32(448))


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


@pytest.mark.parametrize("k", [-7, -1, 3, 9])
@pytest.mark.parametrize("rot", [False, True])
def test_power_of_two_scale_invariance(k, rot):
    x = _rand((2, 3, 200, 64), 1)
    signs = sign_vector(9, 64) if rot else None
    c0, d0 = quantize.quantize_tensor(x, 64, signs)
    c1, d1 = quantize.quantize_tensor(x * np.float32(2.0 ** k), 64, signs)
    assert np.array_equal(c0, c1)
    assert np.array_equal(d1, d0 * np.float32(2.0 ** k))


@pytest.mark.parametrize("rot", [False, True])
def test_dequantisation_error_bound(rot):
    x = _rand((2, 2, 300, 128), 2)
    x[0, 0, 5, 7] = 40.0                      # an outlier inside one block
    signs = sign_vector(3, 128) if rot else None
    codes, descale = quantize.quantize_tensor(x, 128, signs)
    y = quantize.rotate(x, signs).astype(np.float64) if rot else x.astype(np.float64)
    deq = quantize.dequantize(codes, descale, 128)
    ds = np.repeat(descale.astype(np.float64), 128, axis=-1)[..., :300, None]
    # e4m3 rounding: half an ulp is <= 2^-4 relative (normal) or 2^-10 absolute
    # (subnormal, in units of the block scale); the float32 products add ~1e-6 relative
    bound = (2.0 ** -4 * np.abs(y) + 2.0 ** -10 * ds) * (1 + 1e-5)
    assert np.all(np.abs(deq - y) <= bound)
    # every nonzero block reaches the top code (its maximum maps to 448)
    mags = codes & 0x7F
    for blk in range(descale.shape[-1]):
        assert np.all(mags[..., blk * 128:(blk + 1) * 128, :].max(axis=(-2, -1)) == 0x7E)


def test_block_causality_and_ragged_block():
    x = _rand((1, 1, 300, 64), 4)
    c0, d0 = quantize.quantize_tensor(x, 128, sign_vector(1, 64))
    x2 = x.copy()
    x2[..., 256:, :] *= 100                    # only the last (short) block changes
    c1, d1 = quantize.quantize_tensor(x2, 128, sign_vector(1, 64))
    assert np.array_equal(c0[..., :256, :], c1[..., :256, :])
    assert np.array_equal(d0[..., :2], d1[..., :2])
    assert not np.array_equal(d0[..., 2], d1[..., 2])
    # the short block's maximum covers its 44 valid rows only
    y = quantize.rotate(x2, sign_vector(1, 64))[..., 256:, :]
    assert d1[0, 0, 2] == np.abs(y).max() / np.float32(448)


def test_zero_block():
    x = np.zeros((1, 1, 128, 64), dtype=np.float32)
    x[..., 64:, :] = -0.0
    codes, descale = quantize.quantize_tensor(x, 64, None)
    assert np.all(descale == 1.0)
    assert np.all(codes[..., :64, :] == 0x00) and np.all(codes[..., 64:, :] == 0x80)


def test_rotation_cancels_in_qk():
    d = 128
    q = _rand((300, d), 5).astype(np.float64)
    k = _rand((300, d), 6).astype(np.float64)
    s = sign_vector(0x5EED, d).astype(np.float64)
    h = scipy.linalg.hadamard(d).astype(np.float64)
    rq = (q * s) @ h
    rk = (k * s) @ h
    ref = q @ k.T
    got = rq @ rk.T / d
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref)) * d


def test_quantize_qkv_rotates_q_and_k_only():
    q, k, v = (_rand((1, 2, 130, 64), s) for s in (7, 8, 9))
    out = quantize.quantize_qkv(q, k, v, 64, True, 0x5EED)
    signs = sign_vector(0x5EED, 64)
    assert np.array_equal(out[0], quantize.quantize_tensor(q, 64, signs)[0])
    assert np.array_equal(out[1], quantize.quantize_tensor(k, 64, signs)[0])
    assert np.array_equal(out[2], quantize.quantize_tensor(v, 64, None, pow2=True)[0])   # V: power-of-two scales
    assert np.array_equal(out[5], quantize.quantize_tensor(v, 64, None, pow2=True)[1])
    assert out[3].shape == (1, 2, 3) and out[5].dtype == np.float32
    off = quantize.quantize_qkv(q, k, v, 64, False, 0x5EED)
    assert np.array_equal(off[0], quantize.quantize_tensor(q, 64, None)[0])


def test_codes_are_never_nan():
    x = _rand((1, 1, 256, 64), 10, scale=1e30)
    codes, _ = quantize.quantize_tensor(x, 64, None)
    assert not np.any((codes & 0x7F) == 0x7F)
    assert np.all(np.isfinite(e4m3.decode(codes)))


# ---- power-of-two (E8M0) block scales: the smallest 2^e with amax <= 448 * 2^e

@pytest.mark.parametrize("a,e", [
    (448.0, 0), (449.0, 1), (1.0, -8), (1.75, -8), (float(np.nextafter(np.float32(1.75), np.float32(2))), -7),
    (0.0, 0), (2.0 ** -140, -127), (1e38, 118), (224.0, -1), (224.5, 0), (896.0, 1), (3.0e-3, -17),
])
def test_pow2_exponent_worked_examples(a, e):
    # hand-derived: 448 * 2^e >= a > 448 * 2^(e-1); e.g. a = 3e-3: 448 * 2^-17 = 3.42e-3 >= 3e-3 > 1.71e-3
    assert int(quantize.pow2_exponent(np.float32(a))) == e


def test_pow2_exponent_is_the_minimal_integer_brute_force():
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(2000) * 10.0 ** rng.uniform(-30, 30, 2000)).astype(np.float32)
    a = np.abs(a)
    for x, e in zip(a, quantize.pow2_exponent(a)):
        ok = [k for k in range(-127, 128) if float(x) <= 448.0 * 2.0 ** k]
        assert int(e) == max(min(ok), -127)


def test_pow2_block_scales_never_saturate_and_use_the_top_half_of_the_range():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 3, 300, 64)).astype(np.float32) * np.float32(37.5)
    codes, ds = quantize.quantize_tensor(x, 64, None, pow2=True)
    m, e = np.frexp(ds.astype(np.float64))
    assert np.all(m == 0.5)                                    # powers of two
    vals = e4m3.decode(codes)
    for blk in range(ds.shape[-1]):
        v = np.abs(vals[..., blk * 64:(blk + 1) * 64, :]).max(axis=(-2, -1))
        assert np.all(v <= 448) and np.all(v >= 224)           # amax / 2^e in (224, 448]
    # the codes are the e4m3 rounding of x * 2^-e (exact power-of-two scaling)
    inv = np.repeat(1.0 / ds.astype(np.float64), 64, axis=-1)[..., :300]
    ref = e4m3.encode((x.astype(np.float64) * inv[..., None]).astype(np.float32))
    assert np.array_equal(codes, ref)


def test_pow2_zero_block_and_scale_invariance():
    x = np.zeros((1, 128, 64), dtype=np.float32)
    codes, ds = quantize.quantize_tensor(x, 64, None, pow2=True)
    assert np.all(codes == 0) and np.all(ds == 1.0)
    # scaling the input by a power of two moves only the block scales
    rng = np.random.default_rng(9)
    y = rng.standard_normal((1, 128, 64)).astype(np.float32)
    c1, d1 = quantize.quantize_tensor(y, 64, None, pow2=True)
    c2, d2 = quantize.quantize_tensor(y * np.float32(8.0), 64, None, pow2=True)
    assert np.array_equal(c1, c2) and np.array_equal(d2, d1 * 8)

"""Pins of Schraudolph's bit-level exponential (oracle.fastexp) and of the E2
loop's option that uses it: exact values where the method's construction fixes
them (powers of two, linear interpolation between them), the closed-form error
range, monotonicity, saturation, and brute force of the loop on small cases."""

import math

import numpy as np
import pytest

from oracle import attention, e4m3, fastexp
from oracle.fastexp import SIGMA, schraudolph_exp2


def test_sigma_is_schraudolphs_constant():
    # 60801 in units of 2^-20 of the exponent (his double-precision formulation)
    assert SIGMA * 2 ** 20 == 60801


@pytest.mark.parametrize("n", list(range(-125, 128, 7)) + [-126, 0, 1, 127])
def test_exact_at_shifted_integers(n):
    # y = x - sigma an integer -> exponent field n + 127, empty mantissa: exactly 2^n
    assert schraudolph_exp2(n + SIGMA) == 2.0 ** n


@pytest.mark.parametrize("n", [-40, -3, 0, 5, 30])
@pytest.mark.parametrize("k", range(8))
def test_linear_between_powers_of_two(n, k):
    # the mantissa holds the fractional part linearly: 2^n (1 + k/8)
    assert schraudolph_exp2(n + k / 8 + SIGMA) == 2.0 ** n * (1 + k / 8)


def test_error_range_is_the_closed_form():
    x = np.linspace(-30.0, 30.0, 3_000_001)
    rel = schraudolph_exp2(x) / np.exp2(x) - 1
    lo = 2.0 ** -SIGMA - 1                                 # at frac(x - sigma) = 0
    f = 1 / math.log(2) - 1                                # maximiser of (1 + f) 2^-f
    hi = (1 + f) * 2.0 ** (-f - SIGMA) - 1
    # (widened by the float32 rounding of the argument: below 2^-17 relative)
    assert abs(rel.min() - lo) < 2.0 ** -17 and abs(rel.max() - hi) < 2.0 ** -17
    assert -0.0394 < lo < -0.0393 and 0.0196 < hi < 0.0197


def test_float32_argument():
    # the integer comes from the float32 value of 2^23 (x + 127 - sigma): above
    # 2^29 float32 numbers are 64 apart, so an argument of 1064866850 (34 above
    # 1064866816) rounds to 1064866880 before the floor
    x = 1064866850 / 2.0 ** 23 - (127 - SIGMA)
    bits = np.array([schraudolph_exp2(x)], dtype=np.float32).view(np.uint32)[0]
    assert bits == 1064866880
    x = 1064866845 / 2.0 ** 23 - (127 - SIGMA)                     # 29 above: rounds down
    assert np.array([schraudolph_exp2(x)], dtype=np.float32).view(np.uint32)[0] == 1064866816


def test_monotone():
    x = np.linspace(-130.0, 20.0, 2_000_001)
    y = schraudolph_exp2(x)
    assert np.all(np.diff(y) >= 0)


def test_saturation():
    assert 0 < schraudolph_exp2(-126.5 + SIGMA) < 2.0 ** -126        # exponent field 0: subnormal bits
    assert schraudolph_exp2(-127 + SIGMA - 1e-3) == 0.0              # negative integer saturates to 0
    for x in (-128.0 + SIGMA, -200.0, -1e30, -np.inf):
        assert schraudolph_exp2(x) == 0.0
    # the top of the method's range: exponent field 254; above it the integer
    # runs into the exponent's top value and then the sign bit (never reached
    # by the kernel, whose exponents stay <= tau)
    assert schraudolph_exp2(127 + SIGMA) == 2.0 ** 127
    assert math.isinf(schraudolph_exp2(128 + SIGMA))


def _codes(shape, seed, scale):
    x = np.random.default_rng(seed).standard_normal(shape) * scale
    return e4m3.encode(x)


def test_e2_schraudolph_single_block_is_brute_force():
    # one key block and one scale block: the reference m is the row max less
    # the lift (4), r = 1, and the loop must give
    # O = sum_k S(t_k - m) v_k / sum_k S(t_k - m), LSE = ln 2 (m + log2 sum)
    n, d = 64, 64
    q8, k8, v8 = _codes((1, n, d), 1, 40.0), _codes((1, n, d), 2, 40.0), _codes((1, n, d), 3, 40.0)
    qd, kd, vd = np.full((1, 1), 0.02), np.full((1, 1), 0.03), np.full((1, 1), 0.05)
    o, lse = attention.emulated_fp8_attention_tiled(q8, k8, v8, qd, kd, vd, 64, False, False, quantize_p=False,
                                                    bf16_output=False, block_c=64, exp2="schraudolph", lift=4.0)
    q, k, v = e4m3.decode(q8[0]), e4m3.decode(k8[0]), e4m3.decode(v8[0])
    t = (q @ k.T) * (0.02 * 0.03 * math.log2(math.e) / math.sqrt(d))
    m = t.max(axis=1) - 4.0
    w = schraudolph_exp2(t - m[:, None])
    ob = (w @ (v * 0.05)) / w.sum(axis=1)[:, None]
    lb = math.log(2) * (m + np.log2(w.sum(axis=1)))
    assert np.allclose(o[0], ob, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse[0], lb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_e2_schraudolph_fixed_reference_max(causal):
    # the first key block holds a dominant key for every query, and tau is large,
    # so the reference is block 0's max less the lift (4) for the whole row;
    # equal V descales make r = 1.  Then the loop is a plain weighted sum with
    # weights S(t - m0).
    n, d, bc = 256, 64, 64
    rng = np.random.default_rng(7)
    q = rng.standard_normal((n, d)) * 20
    k = rng.standard_normal((n, d)) * 20
    k[0] = q.mean(axis=0) * 8          # key 0 scores high for every query
    q8, k8, v8 = e4m3.encode(q)[None], e4m3.encode(k)[None], _codes((1, n, d), 8, 60.0)
    qd = np.full((1, 4), 0.01)
    kd = np.full((1, 4), 0.01)
    vd = np.full((1, 4), 0.04)
    o, lse = attention.emulated_fp8_attention_tiled(q8, k8, v8, qd, kd, vd, 64, False, causal, tau=1e4,
                                                    quantize_p=False, bf16_output=False, block_c=bc,
                                                    exp2="schraudolph", lift=4.0)
    qq, kk, vv = e4m3.decode(q8[0]), e4m3.decode(k8[0]), e4m3.decode(v8[0]) * 0.04
    t = (qq @ kk.T) * (0.01 * 0.01 * math.log2(math.e) / math.sqrt(d))
    if causal:
        t = np.where(np.arange(n)[None, :] <= np.arange(n)[:, None], t, -np.inf)
    m0 = t[:, :bc].max(axis=1) - 4.0
    w = schraudolph_exp2(t - m0[:, None])
    ob = (w @ vv) / w.sum(axis=1)[:, None]
    lb = math.log(2) * (m0 + np.log2(w.sum(axis=1)))
    assert np.allclose(o[0], ob, rtol=1e-10, atol=1e-10)
    assert np.allclose(lse[0], lb, rtol=1e-10, atol=1e-10)


def test_e2_schraudolph_close_to_exact():
    # the approximation perturbs each weight by at most -3.9% .. +2.0%, so O moves
    # by at most about 6% of max |v| and LSE by at most ln(1.04)
    n, d = 192, 64
    q8, k8, v8 = _codes((1, n, d), 11, 30.0), _codes((1, n, d), 12, 30.0), _codes((1, n, d), 13, 30.0)
    rng = np.random.default_rng(14)
    qd, kd, vd = (rng.uniform(0.005, 0.02, (1, 3)) for _ in range(3))
    kw = dict(quantize_p=False, bf16_output=False)
    oe, le = attention.emulated_fp8_attention_tiled(q8, k8, v8, qd, kd, vd, 64, False, True, **kw)
    os_, ls = attention.emulated_fp8_attention_tiled(q8, k8, v8, qd, kd, vd, 64, False, True, exp2="schraudolph", **kw)
    vmax = np.abs(e4m3.decode(v8)).max() * vd.max()
    assert np.max(np.abs(oe - os_)) <= 0.06 * vmax
    assert np.max(np.abs(le - ls)) <= math.log(1.04)
    assert np.max(np.abs(oe - os_)) > 0          # it is a different function


def test_exp2_mode_is_checked():
    z = np.zeros((1, 64, 64), dtype=np.uint8)
    one = np.ones((1, 1))
    with pytest.raises(ValueError):
        attention.emulated_fp8_attention_tiled(z, z, z, one, one, one, 64, False, False, exp2="fast")

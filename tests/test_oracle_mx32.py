"""Pins of the 32-channel MX block scales of the oracle quantiser
(quantize_tensor(..., pow2=True, group=32)): one E8M0 scale per
(scale_block tokens x 32 channels), FLAMIA 2 Background (MX blocks of 32
elements); hand-derived values, brute-force minimality per group, and the
dequantised attention E1 they define."""

import math

import numpy as np
import pytest

from oracle import attention, e4m3, quantize


def test_hand_derived_groups():
    # d = 64: two groups of 32 channels; two tokens per block
    x = np.zeros((1, 3, 64), np.float32)
    x[0, 0, 3] = 448.0          # group 0 of block 0: amax 448 -> 2^0
    x[0, 1, 40] = -3.0          # group 1 of block 0: amax 3 -> smallest 2^e with 3 <= 448 2^e: e = -7 (3.5 >= 3)
    x[0, 1, 41] = 0.5
    x[0, 2, 0] = 900.0          # block 1 (one token), group 0: 900 <= 448 * 2^2 = 1792, > 896: e = 2 ... 900 > 896 -> e = 2
    # group 1 of block 1 is all zero: 2^0
    codes, ds = quantize.quantize_tensor(x, 2, None, pow2=True, group=32)
    assert ds.shape == (1, 2, 2)
    assert ds[0, 0, 0] == 1.0 and ds[0, 0, 1] == 2.0 ** -7
    assert ds[0, 1, 0] == 4.0 and ds[0, 1, 1] == 1.0
    assert e4m3.decode(codes[0, 0, 3]) == 448.0
    assert e4m3.decode(codes[0, 1, 40]) == -384.0       # -3 * 2^7 = -384 exactly
    assert e4m3.decode(codes[0, 1, 41]) == 64.0
    assert e4m3.decode(codes[0, 2, 0]) == 224.0         # 900 / 4 = 225 -> 224 (spacing 16 in [128, 256))


@pytest.mark.parametrize("d", [64, 128])
def test_each_group_takes_the_smallest_power_of_two(d):
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((2, 3, 300, d)) * np.exp2(rng.integers(-20, 20, size=(2, 3, 1, d)))).astype(np.float32)
    codes, ds = quantize.quantize_tensor(x, 64, None, pow2=True, group=32)
    assert ds.shape == (2, 3, 5, d // 32)
    for b in range(5):
        blk = np.abs(x[..., b * 64:(b + 1) * 64, :]).reshape(2, 3, -1, d // 32, 32).max(axis=(2, 4))
        e = np.log2(ds[..., b, :].astype(np.float64))
        assert np.all(e == np.round(e))
        assert np.all(blk <= 448.0 * 2.0 ** e)
        assert np.all((blk > 224.0 * 2.0 ** e) | (e == -127) | (blk == 0))
    # every code stays inside +-448, no saturation: dequantisation within e4m3's error
    y = quantize.dequantize(codes, ds, 64)
    err = np.abs(y - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) + quantize.dequantize(np.full_like(codes, 1), ds, 64) / 2)


def test_one_group_of_all_channels_is_the_row_rule():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 2, 200, 64)).astype(np.float32) * 7
    c1, d1 = quantize.quantize_tensor(x, 64, None, pow2=True, group=64)
    c2, d2 = quantize.quantize_tensor(x, 64, None, pow2=True)
    assert np.array_equal(c1, c2) and np.array_equal(d1[..., 0], d2)
    with pytest.raises(ValueError):
        quantize.quantize_tensor(x, 64, None, pow2=False, group=32)


def test_groups_isolate_an_outlier_channel():
    # one channel 10^5 times larger: with row scales the other channels fall
    # into e4m3's subnormal range (their codes ~ 448 / 3e5 < 2^-6) and lose
    # their relative precision; with 32-channel groups only its own group does
    rng = np.random.default_rng(6)
    x = rng.standard_normal((1, 1, 128, 128)).astype(np.float32)
    x[..., 5] *= 1e5
    y_row = quantize.dequantize(*quantize.quantize_tensor(x, 128, None, pow2=True), 128)
    y_grp = quantize.dequantize(*quantize.quantize_tensor(x, 128, None, pow2=True, group=32), 128)
    far = np.arange(128) >= 32
    assert np.all(np.abs(y_grp - x)[..., far] <= 2.0 ** -4 * np.abs(x)[..., far] + 2.0 ** -10 * 2.0 ** -6)
    assert np.abs(y_row - x)[..., far].max() > 0.5          # whole values lost to the subnormal range


def test_e1_with_groups_is_attention_of_the_dequantised_inputs():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 2, 150, 64)).astype(np.float32) for _ in range(3))
    qq = quantize.quantize_qkv(q, k, v, 64, True, 3, pow2=True, group=32)
    assert qq[3].shape == (1, 2, 3, 2)
    bars = attention.emulated_fp8_attention_bars(*qq, 64, True, True)
    o, l = attention.attention_fp64(*(quantize.dequantize(c, d, 64) for c, d in zip(qq[:3], qq[3:])), True,
                                    1.0 / (8.0 * 64.0))
    assert np.allclose(bars["o"], o, rtol=1e-12, atol=1e-14) and np.allclose(bars["lse"], l, rtol=1e-12)
    assert np.all(bars["pbar"] > 0) and np.all(np.isfinite(bars["acc_bar"]))

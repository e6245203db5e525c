"""Pins of the oracle's e4m3 decoder and encoder.

The decoder is checked against the closed form of the format and against
torch's independent float8_e4m3fn type; the encoder against torch's CPU cast
(round to nearest even) wherever that cast does not overflow, and against the
saturation rule above 448.
"""

import numpy as np
import pytest
import torch

from oracle import e4m3


def torch_decode(codes):
    t = torch.tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.float().numpy().astype(np.float64)


def torch_encode(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3.decode(codes)
    ref = torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # sign of zero
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_decode_closed_form_landmarks():
    d = e4m3.decode
    assert d(0x38) == 1.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x40) == 2.0 and d(0x30) == 0.5
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert len(e4m3.all_finite_codes()) == 254


def test_encode_decode_roundtrip_every_finite_code():
    codes = e4m3.all_finite_codes()
    assert np.array_equal(e4m3.encode(e4m3.decode(codes)), codes)


def _midpoints():
    pos = np.sort(np.unique(e4m3.decode(e4m3.all_finite_codes())))
    pos = pos[pos >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    return mids.astype(np.float32)


def test_encode_ties_and_neighbours_match_torch():
    mids = _midpoints()
    assert np.all(mids.astype(np.float64) == (mids.astype(np.float64)))  # exact in float32
    xs = np.concatenate([
        mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
    ])
    xs = np.concatenate([xs, -xs]).astype(np.float32)
    assert np.array_equal(e4m3.encode(xs), torch_encode(xs))


def test_encode_random_values_match_torch():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14, np.log2(448.0), size=1_000_000)).astype(np.float32)
    xs = np.where(rng.random(mag.shape) < 0.5, -mag, mag).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    assert np.array_equal(e4m3.encode(xs), torch_encode(xs))


def test_encode_signed_zero_and_underflow():
    xs = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -11, -2.0 ** -11], dtype=np.float32)
    assert list(e4m3.encode(xs)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
    # exactly half the smallest subnormal rounds to even (zero); just above rounds up
    assert e4m3.encode(np.float32(2.0 ** -10)) == 0x00
    assert e4m3.encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01


def test_encode_saturates_above_max():
    xs = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e5, 3e38], dtype=np.float32)
    assert np.all(e4m3.encode(xs) == 0x7E)
    assert np.all(e4m3.encode(-xs) == 0xFE)


def test_encode_is_monotone():
    xs = np.sort(np.random.default_rng(3).uniform(-500, 500, 200_000).astype(np.float32))
    vals = e4m3.decode(e4m3.encode(xs))
    assert np.all(np.diff(vals) >= 0)


def test_encode_rejects_non_finite():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.inf], dtype=np.float32))

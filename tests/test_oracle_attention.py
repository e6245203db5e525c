"""Pins of the oracle's attention: brute force, the running-softmax loop of the
sketch, closed forms, and invariance under the orthogonal rotation."""

import itertools
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import attention, quantize
from oracle.philox import sign_vector


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("n,d", [(1, 4), (3, 4), (6, 8), (5, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force(n, d, causal):
    q, k, v = _rand((n, d), 1), _rand((n, d), 2), _rand((n, d), 3)
    scale = 1 / math.sqrt(d)
    o, lse = attention.attention_fp64(q, k, v, causal, scale)
    ob, lb = attention.brute_force_attention(q.tolist(), k.tolist(), v.tolist(), causal, scale)
    assert np.allclose(o, ob, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("block_c", [1, 3, 64, 128, 200])
@pytest.mark.parametrize("causal", [False, True])
def test_online_softmax_equals_two_pass(block_c, causal):
    n, d = 200, 32
    q, k, v = _rand((n, d), 4, 2.0), _rand((n, d), 5, 2.0), _rand((n, d), 6)
    scale = 1 / math.sqrt(d)
    o, lse = attention.attention_fp64(q, k, v, causal, scale, row_chunk=37)
    oo, lo = attention.online_attention_fp64(q, k, v, causal, scale, block_c)
    assert np.allclose(o, oo, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, lo, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_uniform_weights(causal):
    n, d = 50, 16
    q = np.zeros((n, d))
    k, v = _rand((n, d), 7), _rand((n, d), 8)
    o, lse = attention.reference_attention(q, k, v, causal)
    cnt = np.arange(1, n + 1) if causal else np.full(n, n)
    assert np.allclose(lse, np.log(cnt), rtol=0, atol=1e-14)
    means = np.cumsum(v, axis=0) / cnt[:, None] if causal else np.tile(v.mean(axis=0), (n, 1))
    assert np.allclose(o, means, rtol=0, atol=1e-13)


def test_constant_values_pass_through():
    n, d = 40, 8
    q, k = _rand((n, d), 9, 3.0), _rand((n, d), 10, 3.0)
    c = _rand((d,), 11)
    v = np.tile(c, (n, 1))
    for causal in (False, True):
        o, _ = attention.reference_attention(q, k, v, causal)
        assert np.allclose(o, np.tile(c, (n, 1)), rtol=0, atol=1e-13)


def test_causal_first_row():
    n, d = 30, 8
    q, k, v = _rand((n, d), 12), _rand((n, d), 13), _rand((n, d), 14)
    o, lse = attention.reference_attention(q, k, v, True)
    assert np.array_equal(o[0], v[0])
    assert lse[0] == pytest.approx(q[0] @ k[0] / math.sqrt(d), abs=1e-14)


def test_dominant_key_selects_its_value():
    n, d = 20, 4
    k = np.eye(n, d) * 0
    k[:, 0] = np.arange(n)                       # key j scores proportional to j
    q = np.zeros((n, d))
    q[:, 0] = 60.0 * math.sqrt(d)                # margin between keys >= 60
    v = _rand((n, d), 15)
    o, lse = attention.reference_attention(q, k, v, False)
    assert np.allclose(o, np.tile(v[-1], (n, 1)), atol=1e-20 + math.exp(-50) * np.abs(v).max())
    assert np.allclose(lse, 60.0 * (n - 1), rtol=1e-15)


def test_rotation_invariance_all_signs_d4():
    n, d = 12, 4
    q, k, v = _rand((n, d), 16), _rand((n, d), 17), _rand((n, d), 18)
    h = scipy.linalg.hadamard(d).astype(np.float64)
    o0, l0 = attention.reference_attention(q, k, v, True)
    for signs in itertools.product([-1.0, 1.0], repeat=d):
        s = np.array(signs)
        rq, rk = (q * s) @ h, (k * s) @ h
        o, l = attention.attention_fp64(rq, rk, v, True, 1 / (math.sqrt(d) * d))
        assert np.allclose(o, o0, rtol=1e-12, atol=1e-13)
        assert np.allclose(l, l0, rtol=1e-12, atol=1e-13)


def test_rows_subset_matches_full():
    q, k, v = _rand((2, 3, 100, 16), 19), _rand((2, 3, 100, 16), 20), _rand((2, 3, 100, 16), 21)
    o, l = attention.reference_attention(q, k, v, True)
    rows = [0, 5, 63, 99]
    os_, ls = attention.reference_attention(q, k, v, True, rows=rows)
    assert np.array_equal(o[..., rows, :], os_) and np.array_equal(l[..., rows], ls)


def _grid_inputs(shape, seed):
    """Values that block quantisation reproduces exactly: e4m3 values times 2^k,
    with every block containing +-448 * 2^k."""
    from oracle import e4m3
    rng = np.random.default_rng(seed)
    codes = rng.choice(e4m3.all_finite_codes(), size=shape)
    x = e4m3.decode(codes)
    x[..., ::64, 0] = 448.0
    return (x * 2.0 ** -6).astype(np.float32)


def test_emulated_attention_is_reference_on_exact_inputs():
    shape = (1, 2, 128, 64)
    q, k, v = (_grid_inputs(shape, s) for s in (22, 23, 24))
    q8, k8, v8, qd, kd, vd = quantize.quantize_qkv(q, k, v, 64, False, 0)
    for causal in (False, True):
        oe, le = attention.emulated_fp8_attention(q8, k8, v8, qd, kd, vd, 64, False, causal)
        orf, lr = attention.reference_attention(q, k, v, causal)
        assert np.array_equal(oe, orf) and np.array_equal(le, lr)


def test_emulated_attention_with_rotation_tracks_reference():
    shape = (1, 2, 256, 64)
    q, k, v = (_rand(shape, s).astype(np.float32) for s in (25, 26, 27))
    q8, k8, v8, qd, kd, vd = quantize.quantize_qkv(q, k, v, 64, True, 0x5EED)
    oe, le = attention.emulated_fp8_attention(q8, k8, v8, qd, kd, vd, 64, True, False)
    orf, lr = attention.reference_attention(q, k, v, False)
    rel = np.sqrt(np.mean((oe - orf) ** 2)) / np.sqrt(np.mean(orf ** 2))
    assert rel < 0.08                           # e4m3 carries ~2^-4 relative error
    assert np.max(np.abs(le - lr)) < 0.1
    # a dropped 1/d would scale scores by 64: the LSE would be far off
    o_bad, l_bad = attention.attention_fp64(quantize.dequantize(q8, qd, 64), quantize.dequantize(k8, kd, 64),
                                            quantize.dequantize(v8, vd, 64), False, 1 / math.sqrt(64))
    assert np.max(np.abs(l_bad - lr)) > 1.0

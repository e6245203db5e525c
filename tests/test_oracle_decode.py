"""Pins of the FP8 K/V-cache decode oracle (oracle.decode): against masked
exact attention of the dequantised cache for every split (the merge is exact),
against E2 where the two coincide (one range, equal V descales), grouped-query
heads against repeated K/V heads, and the cache beyond each sequence's length
unused."""

import math

import numpy as np
import pytest

from oracle import attention, decode, e4m3


def _cache(rng, B, Hq, Hkv, Sq, Ncap, D, sb, spread=(0.002, 0.02)):
    q8 = e4m3.encode(rng.standard_normal((B, Hq, Sq, D)) * 30)
    k8 = e4m3.encode(rng.standard_normal((B, Hkv, Ncap, D)) * 30)
    v8 = e4m3.encode(rng.standard_normal((B, Hkv, Ncap, D)) * 30)
    nb = -(-Ncap // sb)
    qd = rng.uniform(*spread, (B, Hq, 1))
    kd = rng.uniform(*spread, (B, Hkv, nb))
    vd = rng.uniform(*spread, (B, Hkv, nb))
    return q8, qd, k8, v8, kd, vd


def _masked_reference(q8, qd, k8, v8, kd, vd, seqlens, sb, hadamard, causal):
    """Exact float64 attention of the dequantised values, positions and grouping written out."""
    B, Hq, Sq, D = q8.shape
    Hkv = k8.shape[1]
    G = Hq // Hkv
    scale = 1 / math.sqrt(D) / (D if hadamard else 1)
    o = np.zeros((B, Hq, Sq, D))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        L = int(seqlens[b])
        for h in range(Hq):
            g = h // G
            q = e4m3.decode(q8[b, h]) * qd[b, h, 0]
            k = e4m3.decode(k8[b, g, :L]) * np.repeat(kd[b, g], sb)[:L, None]
            v = e4m3.decode(v8[b, g, :L]) * np.repeat(vd[b, g], sb)[:L, None]
            s = (q @ k.T) * scale
            if causal:
                pos = L - Sq + np.arange(Sq)
                s = np.where(np.arange(L)[None, :] <= pos[:, None], s, -np.inf)
            mx = s.max(axis=1)
            w = np.exp(s - mx[:, None])
            o[b, h] = (w @ v) / w.sum(axis=1)[:, None]
            lse[b, h] = mx + np.log(w.sum(axis=1))
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("split", [64, 128, 192, 4096])
def test_without_p_rounding_every_split_is_exact_attention(causal, split):
    rng = np.random.default_rng(split + causal)
    B, Hq, Hkv, Sq, Ncap, D, sb = 2, 4, 2, 3, 700, 64, 128
    args = _cache(rng, B, Hq, Hkv, Sq, Ncap, D, sb)
    seqlens = np.array([700, 129])
    o, lse = decode.emulated_fp8_decode(*args, seqlens, sb, True, causal, split, quantize_p=False, bf16_output=False)
    ob, lb = _masked_reference(*args, seqlens, sb, True, causal)
    assert np.allclose(o, ob, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, lb, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_one_range_is_e2(causal):
    # Sq = L makes the decode a full attention call (query i at position i):
    # one range is then the dense loop
    rng = np.random.default_rng(3)
    B, H, L, D, sb = 1, 2, 300, 64, 64
    q8, qd, k8, v8, kd, vd = _cache(rng, B, H, H, L, L, D, sb)
    vd[:] = 0.01
    qd_blocks = np.repeat(qd, -(-L // sb), axis=2)        # the same descale for every query block
    o, lse = decode.emulated_fp8_decode(q8, qd, k8, v8, kd, vd, [L], sb, True, causal, 1024)
    o2, l2 = attention.emulated_fp8_attention_tiled(q8, k8, v8, qd_blocks, kd, vd, sb, True, causal)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, l2, rtol=1e-12, atol=1e-12)


def test_grouped_queries_read_their_kv_head():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, Sq, Ncap, D, sb = 1, 6, 2, 2, 400, 128, 128
    q8, qd, k8, v8, kd, vd = _cache(rng, B, Hq, Hkv, Sq, Ncap, D, sb)
    G = Hq // Hkv
    rep = lambda x: np.repeat(x, G, axis=1)
    a = decode.emulated_fp8_decode(q8, qd, k8, v8, kd, vd, [333], sb, False, True, 128)
    b = decode.emulated_fp8_decode(q8, qd, rep(k8), rep(v8), rep(kd), rep(vd), [333], sb, False, True, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_cache_past_the_length_is_unused():
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Sq, Ncap, D, sb = 2, 2, 1, 1, 512, 64, 64
    q8, qd, k8, v8, kd, vd = _cache(rng, B, Hq, Hkv, Sq, Ncap, D, sb)
    seqlens = [200, 512]
    a = decode.emulated_fp8_decode(q8, qd, k8, v8, kd, vd, seqlens, sb, True, False, 128)
    k2, v2, kd2, vd2 = k8.copy(), v8.copy(), kd.copy(), vd.copy()
    k2[0, :, 200:] = 0x7E
    v2[0, :, 200:] = 0x7E
    kd2[0, :, 4:] = 1e3          # block 3 holds tokens 192..255: it stays
    vd2[0, :, 4:] = 1e3
    b = decode.emulated_fp8_decode(q8, qd, k2, v2, kd2, vd2, seqlens, sb, True, False, 128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_changes_only_p_rounding():
    # with P rounded, different splits differ only by P's e4m3 rounding at
    # different reference maxima: within a few e4m3 steps of P, in relative terms
    rng = np.random.default_rng(6)
    args = _cache(rng, 1, 2, 2, 1, 1000, 64, 128)
    a, la = decode.emulated_fp8_decode(*args, [1000], 128, True, False, 64, bf16_output=False)
    b, lb = decode.emulated_fp8_decode(*args, [1000], 128, True, False, 1024, bf16_output=False)
    assert np.allclose(la, lb, rtol=1e-12)                 # l never sees the rounding
    vmax = np.abs(e4m3.decode(args[3])).max() * args[5].max()
    assert 0 < np.max(np.abs(a - b)) < 0.07 * vmax


def test_arguments_are_checked():
    rng = np.random.default_rng(7)
    args = _cache(rng, 1, 2, 2, 4, 256, 64, 64)
    with pytest.raises(ValueError):
        decode.emulated_fp8_decode(*args, [256], 64, True, False, 100)     # split not a multiple of 64
    with pytest.raises(ValueError):
        decode.emulated_fp8_decode(*args, [3], 64, True, False, 128)       # fewer tokens than queries
    with pytest.raises(ValueError):
        decode.emulated_fp8_decode(*args, [257], 64, True, False, 128)     # past the cache
